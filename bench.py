"""Benchmark of the block-FP8 linear-layer hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input.
Workloads (--workload):
  dense  (default) 8B-shaped dense layer at M = 8192 tokens: per-step
         recalibration of the layer's four weights (128x128 quantizer), the
         1x128 quantization of each GEMM input, and the four block-scaled
         GEMMs QKV (K 4096, N 6144), gate+up (K 4096, N 28672),
         down (K 14336, N 4096), o_proj (K 4096, N 4096).
  recal  per-step recalibration of 32 layers x 4 weights, EXACT then POW2.
  decode rollout decode: M in {1, 16, 64, 256} against the gate+up and down
         weights, through fp8_block_linear from bf16 activations (one launch
         that quantizes inside the GEMM for M <= 16 where the W tiles are 32 or
         64 rows, i.e. gate+up); the separate quantizer and GEMM calls are
         timed after the step for comparison.
  train  training backward of the dense layer: W and W^T codes from one
         batched recalibration launch; per layer the quantization of dY, the
         data-gradient GEMM dX = dY W, the quantization of dY^T and X^T along
         the tokens and the weight-gradient GEMM dW = dY^T X.
  moe    MoE layer: 128 experts, hidden 2048, expert FFN 768, 8192 tokens
         routed top-8: expert-weight recalibration, quantization of the
         gate+up and down inputs, the two grouped GEMMs.
Prints ONE JSON line.  `value` is GEMM TFLOP/s over the whole step
(quantizers included) except for `recal` (GB/s).  Per-kernel times come from
HIP events recorded on the stream the library launches on (torch's current
stream, whose handle every call passes to the library).

Tool modes (no GPU work of their own):
  --copy-calibration   after the timed steps, copy a 1 GiB buffer three times
                       (a plain copy kernel of known size, the reference for
                       scaling rocprofv3 FETCH_SIZE / WRITE_SIZE);
  --summarize-pmc FETCH_DB WRITE_DB  turn two rocprofv3 --pmc databases of
                       `bench.py --copy-calibration` into the traffic record
                       profiles/<kernel>_traffic.json that the roofline reads.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-FP8 GEMM TFLOP/s (% of FP8 MFMA peak); quantizer GB/s (% of HBM peak)"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)

DENSE = [("qkv", 6144, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336), ("o_proj", 4096, 4096)]
GEMM_SRC = os.path.join(ROOT, "block_scaled_fp8_x128_amd", "csrc", "fp8bs_gemm.hip")
QUANT_SRC = os.path.join(ROOT, "block_scaled_fp8_x128_amd", "csrc", "fp8bs_quant.hip")
COPY_BYTES = 1 << 30

# Dominant kernel of each workload: (kernel-name prefix in a rocprofv3 trace,
# source file, traffic record under profiles/).
DOMINANT = {
    "dense": ("fp8bs::gemm_dma_kernel<256, 256, 4, 2, false, false, false, false, false>", GEMM_SRC,
              "gemm_dma_256x256_dense_m8192_traffic.json"),
    "recal": ("fp8bs::quant_w_kernel<0>", QUANT_SRC, "quant_w_recal_32layers_traffic.json"),
    # the grouped gate+up call: its row-tile table, the 256-row pass and the short-tile pass
    "moe": ("fp8_block_grouped_gemm gate+up", GEMM_SRC, "grouped_gemm_moe_gate_up_traffic.json"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def src_hash(path: str) -> str:
    return hashlib.sha256(open(path, "rb").read()).hexdigest()[:16]


# ---------------------------------------------------------------------------
# timing
# ---------------------------------------------------------------------------

class KernelTimer:
    """Per-call HIP-event timing on torch's current stream (the library's stream)."""

    def __init__(self):
        self.pairs = {}

    def run(self, name, fn):
        import torch
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        out = fn()
        b.record()
        self.pairs.setdefault(name, []).append((a, b))
        return out

    def avg_ms(self, name):
        ps = self.pairs[name]
        return sum(a.elapsed_time(b) for a, b in ps) / len(ps)

    def spread(self, name):
        """(median, min) of the timed launches of `name`, in ms."""
        v = sorted(a.elapsed_time(b) for a, b in self.pairs[name])
        n = len(v)
        med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
        return med, v[0]

    def reset(self):
        self.pairs = {}


def timed_loop(step, steps, warmup, timer):
    import torch
    for _ in range(warmup):
        step(None)
    torch.cuda.synchronize()
    timer.reset()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timer)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def maybe(timer, name, fn):
    return timer.run(name, fn) if timer is not None else fn()


def bf16_dev(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def hbm_entry(ms, nbytes):
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def mfma_entry(ms, flops):
    tf = flops / (ms * 1e-3) / 1e12
    return {"ms": round(ms, 4), "TFLOP/s": round(tf, 1), "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}


def traffic_for(workload):
    """HBM bytes per launch of the dominant kernel from its committed
    rocprofv3 record, or None if there is none or the kernel source changed."""
    if workload not in DOMINANT:
        return None, None
    _, src, fname = DOMINANT[workload]
    path = os.path.join(ROOT, "profiles", fname)
    if not os.path.exists(path):
        return None, None
    rec = json.load(open(path))
    if rec.get("source_sha256_16") != src_hash(src):
        return None, "stale: %s was taken before the last change of %s" % (fname, os.path.basename(src))
    return rec["hbm_bytes_per_launch"], "profiles/" + fname


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def dense_workload(fp8bs, dev, mode):
    # POW2 scales go to the entry points that apply them through the matrix cores
    gemm = fp8bs.fp8_block_gemm_pow2 if mode else fp8bs.fp8_block_gemm
    grouped = fp8bs.fp8_block_grouped_gemm_pow2 if mode else fp8bs.fp8_block_grouped_gemm
    import synth
    import torch
    M = 8192
    bufs = []
    for i, (name, N, K) in enumerate(DENSE):
        log("generating %s: X [%d, %d], W [%d, %d]" % (name, M, K, N, K))
        x = bf16_dev(synth.activations(M, K, sub=synth.SUB_X + 10 * i), dev)
        w = bf16_dev(synth.weights(N, K, sub=synth.sub_layer(i)), dev)
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        xs = torch.empty((M, K // 128), dtype=torch.float32, device=dev)
        wq = torch.empty((N, K), dtype=torch.uint8, device=dev)
        ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        bufs.append(dict(name=name, M=M, N=N, K=K, x=x, w=w, xq=xq, xs=xs, wq=wq, ws=ws, y=y))

    w_all = [b["w"] for b in bufs]
    out_all = [(b["wq"], b["ws"]) for b in bufs]

    def step(timer):
        # the step's recalibration: all four weights in one batched launch
        maybe(timer, "quant_w_all", lambda: fp8bs.quant_w_128x128_batched(w_all, mode, outs=out_all))
        for b in bufs:
            maybe(timer, "quant_act_" + b["name"], lambda: fp8bs.quant_act_1x128(b["x"], mode, out=(b["xq"], b["xs"])))
            maybe(timer, "gemm_" + b["name"],
                  lambda: gemm(b["xq"], b["xs"], b["wq"], b["ws"], out=b["y"]))

    flops = sum(2.0 * b["M"] * b["N"] * b["K"] for b in bufs)
    return step, bufs, flops


def train_workload(fp8bs, dev, mode):
    """Backward data gradients of the same four layers: dX [M, K] = dY [M, N] W [N, K]."""
    gemm = fp8bs.fp8_block_gemm_pow2 if mode else fp8bs.fp8_block_gemm
    import synth
    import torch
    M = 8192
    bufs = []
    for i, (name, N, K) in enumerate(DENSE):
        log("generating %s: dY [%d, %d], W [%d, %d]" % (name, M, N, N, K))
        dy = bf16_dev(synth.activations(M, N, sub=synth.SUB_DY + 10 * i), dev)
        w = bf16_dev(synth.weights(N, K, sub=synth.sub_layer(i)), dev)
        outs = (torch.empty((N, K), dtype=torch.uint8, device=dev),
                torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev),
                torch.empty((K, N), dtype=torch.uint8, device=dev),
                torch.empty((K // 128, N // 128), dtype=torch.float32, device=dev))
        x = bf16_dev(synth.activations(M, K, sub=synth.SUB_X + 10 * i), dev)
        dyq = torch.empty((M, N), dtype=torch.uint8, device=dev)
        dys = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
        dx = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
        # weight gradient: dY^T and X^T quantized along the tokens, dW [N, K]
        dyt = (torch.empty((N, M), dtype=torch.uint8, device=dev),
               torch.empty((N, M // 128), dtype=torch.float32, device=dev))
        xt = (torch.empty((K, M), dtype=torch.uint8, device=dev),
              torch.empty((K, M // 128), dtype=torch.float32, device=dev))
        dw = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
        # the data-gradient GEMM runs with the forward (N, K) swapped: output width K, reduction over N
        bufs.append(dict(name=name, M=M, N=K, K=N, dy=dy, w=w, x=x, outs=outs, dyq=dyq, dys=dys, dx=dx,
                         dyt=dyt, xt=xt, dw=dw))

    w_all = [b["w"] for b in bufs]
    out_all = [b["outs"] for b in bufs]

    def step(timer):
        # the step's recalibration for training: W and W^T codes from one read of each weight
        maybe(timer, "quant_w_all", lambda: fp8bs.quant_w_128x128_dual_batched(w_all, mode, outs=out_all))
        for b in bufs:
            # dY quantized along its rows (data gradient) and along the tokens (weight gradient), one read
            maybe(timer, "quant_act_dual_dy_" + b["name"],
                  lambda: fp8bs.quant_act_1x128_dual(b["dy"], mode, out=(b["dyq"], b["dys"]) + b["dyt"]))
            maybe(timer, "gemm_" + b["name"],
                  lambda: gemm(b["dyq"], b["dys"], b["outs"][2], b["outs"][3], out=b["dx"]))
            maybe(timer, "quant_act_t_x_" + b["name"], lambda: fp8bs.quant_act_1x128_t(b["x"], mode, out=b["xt"]))
            maybe(timer, "wgrad_" + b["name"],
                  lambda: fp8bs.fp8_block_gemm_1x128(b["dyt"][0], b["dyt"][1], b["xt"][0], b["xt"][1], out=b["dw"]))

    # data and weight gradients: twice the forward FLOPs
    flops = sum(4.0 * b["M"] * b["N"] * b["K"] for b in bufs)
    return step, bufs, flops


def summarize_train(bufs, timer):
    """The data-gradient half as summarize_dense, plus the weight-gradient GEMMs and
    the transposing quantizers; the roofline object covers whichever GEMM kernel
    takes more of the step."""
    kernels, roof = summarize_dense(bufs, timer, dual=True)
    w_ms, w_flops = [], []
    for b in bufs:
        M, N, K = b["M"], b["N"], b["K"]   # (tokens, forward K, forward N)
        t = timer.avg_ms("wgrad_" + b["name"])
        kernels["wgrad_" + b["name"]] = mfma_entry(t, 2.0 * M * N * K)
        w_ms.append(t)
        w_flops.append(2.0 * M * N * K)
        # dY [M, K] (K = the forward N here): bf16 read once, two code sets and two scale sets written
        kernels["quant_act_dual_dy_" + b["name"]] = hbm_entry(
            timer.avg_ms("quant_act_dual_dy_" + b["name"]), M * K * 4 + (M * K // 128) * 8)
        kernels["quant_act_t_x_" + b["name"]] = hbm_entry(
            timer.avg_ms("quant_act_t_x_" + b["name"]), M * N * 3 + (M * N // 128) * 4)
    d_ms = roof["avg_launch_ms"] * len(bufs)
    if sum(w_ms) > d_ms:
        mean_ms, mean_flops = sum(w_ms) / len(w_ms), sum(w_flops) / len(w_flops)
        ach = mean_flops / (mean_ms * 1e-3) / 1e12
        roof = {"kernel": "fp8bs::gemm_dma_kernel<256, 256, 4, 2, false, false, false, false, true> (weight "
                          "gradients of QKV, gate+up, down, o_proj over 8192 tokens)", "bound": "mfma",
                "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": None,
                "algorithmic_flop_per_launch": mean_flops, "avg_launch_ms": round(mean_ms, 4),
                "traffic_source": None}
    return kernels, roof


def summarize_dense(bufs, timer, dual=False):
    kernels = {}
    gemm_ms, gemm_flops = [], []
    for b in bufs:
        M, N, K = b["M"], b["N"], b["K"]
        t = timer.avg_ms("gemm_" + b["name"])
        kernels["gemm_" + b["name"]] = mfma_entry(t, 2.0 * M * N * K)
        gemm_ms.append(t)
        gemm_flops.append(2.0 * M * N * K)
        if "quant_act_" + b["name"] in timer.pairs:
            kernels["quant_act_" + b["name"]] = hbm_entry(timer.avg_ms("quant_act_" + b["name"]),
                                                          M * K * 3 + (M * K // 128) * 4)
    # bf16 read, codes written (twice for the dual form: W and W^T), one fp32 per block (twice)
    wb = 4 if dual else 3
    kernels["quant_w_all"] = hbm_entry(timer.avg_ms("quant_w_all"),
                                       sum(b["N"] * b["K"] * wb + (b["N"] * b["K"] // 16384) * 4 * (wb - 2)
                                           for b in bufs))
    # The four GEMMs run one kernel (the 256 x 256 persistent block-scaled
    # GEMM): per launch, mean algorithmic FLOP / mean duration.
    mean_ms = sum(gemm_ms) / len(gemm_ms)
    mean_flops = sum(gemm_flops) / len(gemm_flops)
    ach = mean_flops / (mean_ms * 1e-3) / 1e12
    traffic, tsrc = traffic_for("dense")
    what = "data gradients of " if dual else ""
    roof = {"kernel": DOMINANT["dense"][0] + " (%sQKV, gate+up, down, o_proj at M=8192)" % what, "bound": "mfma",
            "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
            "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": traffic,
            "algorithmic_flop_per_launch": mean_flops, "avg_launch_ms": round(mean_ms, 4),
            "traffic_source": tsrc}
    return kernels, roof


def cpu_baseline_dense(target_s=12.0):
    """The oracle GEMM (exact per-block sums, fp64 scales) on a bounded sample
    of the gate+up GEMM: the first R rows of Y, R sized for ~target_s."""
    import oracle
    import synth
    N, K = 28672, 4096
    threads = oracle.max_threads()
    w = synth.weights(N, K, sub=synth.sub_layer(1))
    wq, ws = oracle.quant_w_128x128(w)
    rows = 2
    while True:
        x = synth.activations(rows, K, sub=synth.SUB_X + 10)
        xq, xs = oracle.quant_act_1x128(x)
        t0 = time.perf_counter()
        oracle.gemm(xq, xs, wq, ws)
        dt = time.perf_counter() - t0
        if dt >= target_s or rows >= 8192:
            break
        rows = min(8192, max(rows * 2, int(rows * target_s / max(dt, 1e-3) * 1.05)))
    tflops = 2.0 * rows * N * K / dt / 1e12
    return {"value": tflops, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "gate+up GEMM (N 28672, K 4096), first %d of 8192 rows, %.1f s wall" % (rows, dt)}


def recal_workload(fp8bs, dev):
    import synth
    import torch
    shapes = [(6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336)]
    log("generating 32 layers x 4 bf16 weights on the device (seeded torch generator)")
    ws_in, outs = [], []
    for layer in range(32):
        g = torch.Generator(device=dev)
        g.manual_seed(synth.sub_layer(layer))
        for (N, K) in shapes:
            w = (torch.randn((N, K), generator=g, device=dev, dtype=torch.float32) * 0.02).to(torch.bfloat16)
            ws_in.append(w)
            outs.append((torch.empty((N, K), dtype=torch.uint8, device=dev),
                         torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev)))
    elems = sum(w.numel() for w in ws_in)

    def step(timer):
        for mode, name in ((0, "recal_exact"), (1, "recal_pow2")):
            maybe(timer, name, lambda: fp8bs.quant_w_128x128_batched(ws_in, mode, outs=outs))

    nbytes = elems * 3 + (elems // 16384) * 4
    return step, nbytes


def cpu_baseline_recal(target_s=12.0):
    """The oracle's 128x128 quantizer on a bounded sample of the recalibration:
    whole 28672 x 4096 weight tensors until ~target_s."""
    import oracle
    import synth
    w = synth.weights(28672, 4096, sub=synth.sub_layer(0))
    n, t = 0, 0.0
    while t < target_s and n < 16:
        t0 = time.perf_counter()
        oracle.quant_w_128x128(w, 0)
        t += time.perf_counter() - t0
        n += 1
    nbytes = n * (w.size * 3 + (w.size // 16384) * 4)
    return {"value": nbytes / t / 1e9, "unit": "GB/s", "cores": oracle.max_threads(), "kind": "oracle",
            "sample": "%d quantizations (EXACT) of one 28672 x 4096 weight, %.1f s wall" % (n, t)}


def decode_workload(fp8bs, dev, mode):
    # POW2 scales go to the entry points that apply them through the matrix cores
    gemm = fp8bs.fp8_block_gemm_pow2 if mode else fp8bs.fp8_block_gemm
    linear = fp8bs.fp8_block_linear_pow2 if mode else fp8bs.fp8_block_linear
    import synth
    import torch
    pairs = []
    for wname, N, K in (("gate_up", 28672, 4096), ("down", 4096, 14336)):
        log("generating %s weights [%d, %d]" % (wname, N, K))
        # five weight copies rotated over the calls, so that the 256 MB
        # infinity cache never holds the weights a GEMM reads
        copies = []
        for c in range(5):
            wq, ws = fp8bs.quant_w_128x128(bf16_dev(synth.weights(N, K, sub=synth.sub_layer(40 + c)), dev), mode)
            copies.append((wq, ws))
        for j, M in enumerate((1, 16, 64, 256)):
            x = bf16_dev(synth.activations(M, K, sub=synth.SUB_X + M), dev)
            pairs.append(dict(name="%s_m%d" % (wname, M), M=M, N=N, K=K, x=x, copies=copies, j=j,
                              xq=torch.empty((M, K), dtype=torch.uint8, device=dev),
                              xs=torch.empty((M, K // 128), dtype=torch.float32, device=dev),
                              y=torch.empty((M, N), dtype=torch.bfloat16, device=dev),
                              ws_buf=torch.empty(max(1, fp8bs.gemm_workspace_size(M, N, K)), dtype=torch.uint8,
                                                 device=dev),
                              lin_buf=torch.empty(max(1, fp8bs.linear_workspace_size(M, N, K)), dtype=torch.uint8,
                                                  device=dev)))
    it = [0]

    def step(timer):
        # the linear layer from bf16 activations: one launch for M <= 16 (X
        # quantized inside the weight-streaming GEMM or the one-row GEMV),
        # quantizer + GEMM above.  Each call of a step reads its own weight
        # copy: between two reads of a copy, more than the 256 MB cache's
        # worth of other weights passes
        c = it[0]
        it[0] += 1
        for p in pairs:
            wq, ws = p["copies"][(c + p["j"]) % 5]
            maybe(timer, "linear_" + p["name"],
                  lambda p=p, wq=wq, ws=ws: linear(p["x"], wq, ws, out=p["y"], workspace=p["lin_buf"]))

    def separate(timer, reps):
        # the same layer as two separate calls, timed apart (reported beside the step)
        for r in range(reps):
            for p in pairs:
                wq, ws = p["copies"][(r + p["j"]) % 5]
                maybe(timer, "quant_" + p["name"],
                      lambda p=p: fp8bs.quant_act_1x128(p["x"], mode, out=(p["xq"], p["xs"])))
                maybe(timer, "gemm_" + p["name"],
                      lambda p=p, wq=wq, ws=ws: gemm(p["xq"], p["xs"], wq, ws, out=p["y"], workspace=p["ws_buf"]))

    flops = sum(2.0 * p["M"] * p["N"] * p["K"] for p in pairs)
    return step, separate, pairs, flops


T_TOKENS = 8192  # tokens of the MoE layer (each routed to 8 of 128 experts)


def moe_workload(fp8bs, dev, mode):
    # POW2 scales go to the entry points that apply them through the matrix cores
    gemm = fp8bs.fp8_block_gemm_pow2 if mode else fp8bs.fp8_block_gemm
    grouped = fp8bs.fp8_block_grouped_gemm_pow2 if mode else fp8bs.fp8_block_grouped_gemm
    import synth
    import torch
    E, H, F, T, TOPK = 128, 2048, 768, T_TOKENS, 8
    row_token, offs = synth.moe_routing(T, E, TOPK)
    Mt = int(offs[-1])
    log("MoE: %d routed rows, per-expert rows min %d max %d" % (Mt, int(np.diff(offs).min()), int(np.diff(offs).max())))
    x_tok = synth.activations(T, H, sub=synth.SUB_X)
    # the dispatch: each routed row reads its token's row (quantized on the way, in expert order)
    xt = bf16_dev(x_tok, dev)
    rows_d = torch.from_numpy(np.ascontiguousarray(row_token, dtype=np.int32)).to(dev)
    w1 = bf16_dev(synth.expert_weights(E, 2 * F, H, sub=synth.SUB_W).reshape(E * 2 * F, H), dev)
    w2 = bf16_dev(synth.expert_weights(E, H, F, sub=synth.SUB_W + 1).reshape(E * H, F), dev)
    offs_d = torch.from_numpy(offs).to(dev)
    b = dict(
        x1q=torch.empty((Mt, H), dtype=torch.uint8, device=dev), x1s=torch.empty((Mt, H // 128), dtype=torch.float32,
                                                                                  device=dev),
        x2q=torch.empty((Mt, F), dtype=torch.uint8, device=dev), x2s=torch.empty((Mt, F // 128), dtype=torch.float32,
                                                                                  device=dev),
        w1q=torch.empty((E * 2 * F, H), dtype=torch.uint8, device=dev),
        w1s=torch.empty((E * 2 * F // 128, H // 128), dtype=torch.float32, device=dev),
        w2q=torch.empty((E * H, F), dtype=torch.uint8, device=dev),
        w2s=torch.empty((E * H // 128, F // 128), dtype=torch.float32, device=dev),
        y1=torch.empty((Mt, 2 * F), dtype=torch.bfloat16, device=dev),
        y2=torch.empty((Mt, H), dtype=torch.bfloat16, device=dev),
        wk1=torch.empty(max(1, fp8bs.grouped_workspace_size(E, Mt, 2 * F, H)), dtype=torch.uint8, device=dev),
        wk2=torch.empty(max(1, fp8bs.grouped_workspace_size(E, Mt, H, F)), dtype=torch.uint8, device=dev))

    def step(timer):
        maybe(timer, "quant_w_experts", lambda: fp8bs.quant_w_128x128_batched([w1, w2], mode,
                                                                               outs=[(b["w1q"], b["w1s"]),
                                                                                     (b["w2q"], b["w2s"])]))
        maybe(timer, "quant_act_gather_gate_up", lambda: fp8bs.quant_act_1x128_gather(xt, rows_d, mode,
                                                                                    out=(b["x1q"], b["x1s"])))
        maybe(timer, "grouped_gate_up", lambda: grouped(
            b["x1q"], b["x1s"], b["w1q"].view(E, 2 * F, H), b["w1s"].view(E, 2 * F // 128, H // 128), offs_d,
            out=b["y1"], workspace=b["wk1"]))
        # the gated activation of the gate+up output, quantized for the down projection
        maybe(timer, "swiglu_quant_down", lambda: fp8bs.swiglu_quant_1x128(b["y1"], mode, out=(b["x2q"], b["x2s"])))
        maybe(timer, "grouped_down", lambda: grouped(
            b["x2q"], b["x2s"], b["w2q"].view(E, H, F), b["w2s"].view(E, H // 128, F // 128), offs_d, out=b["y2"],
            workspace=b["wk2"]))

    shapes = {"gate_up": (Mt, 2 * F, H), "down": (Mt, H, F)}
    flops = sum(2.0 * m * n * k for m, n, k in shapes.values())
    return step, shapes, flops, E


# ---------------------------------------------------------------------------
# rocprofv3 counter records
# ---------------------------------------------------------------------------

def _pmc_means(db, counter):
    """Mean per-dispatch value of `counter` for every kernel name in a rocprofv3 database."""
    import sqlite3
    c = sqlite3.connect(db)
    per = {}
    for kname, val, did in c.execute("select kernel_name, value, dispatch_id from counters_collection "
                                     "where counter_name = ?", (counter,)):
        per.setdefault(kname, {}).setdefault(did, 0.0)
        per[kname][did] += val
    return {k: (sum(v.values()) / len(v), len(v)) for k, v in per.items()}


def _pmc_dispatches(db, counter):
    """[(dispatch_id, kernel_name, value)] in dispatch order."""
    import sqlite3
    c = sqlite3.connect(db)
    per = {}
    for kname, val, did in c.execute("select kernel_name, value, dispatch_id from counters_collection "
                                     "where counter_name = ?", (counter,)):
        k = per.setdefault(did, [kname, 0.0])
        k[1] += val
    return sorted((d, k, v) for d, (k, v) in per.items())


def _copy_calibration(db, counter):
    """Mean counter value of the calibration copies: the runtime's copyBuffer
    dispatches within a factor of two of the largest one."""
    vals = [v for _, k, v in _pmc_dispatches(db, counter) if "copybuffer" in k.lower()]
    if not vals:
        raise SystemExit("no calibration copy in the counter database")
    big = [v for v in vals if v >= 0.5 * max(vals)]
    return sum(big) / len(big)


def _grouped_gate_up_calls(db, counter):
    """Mean value per grouped gate+up call of the MoE step, and the number of
    calls: the table and GEMM dispatches that follow the dispatch quantizer
    (the down call follows the gated activation instead)."""
    calls, cur, after_quant = [], None, False
    for _, k, v in _pmc_dispatches(db, counter):
        if "grouped_tile_table_kernel" in k:
            cur = [v] if after_quant else None
            if cur is not None:
                calls.append(cur)
            after_quant = False
        elif "gemm_dma_kernel" in k and cur is not None:
            cur.append(v)
        else:
            cur = None
            after_quant = "quant_act_kernel" in k or "quant_act_gather_kernel" in k
    if not calls:
        raise SystemExit("no grouped gate+up call found in the counter database")
    return sum(sum(c) for c in calls) / len(calls), len(calls)


def summarize_pmc(fetch_db, write_db, workload, command, out=None):
    """Write the traffic record of `workload`'s dominant kernel (to profiles/
    unless `out` names another file) and return it."""
    kprefix, src, fname = DOMINANT[workload]
    fetch = _pmc_means(fetch_db, "FETCH_SIZE")
    write = _pmc_means(write_db, "WRITE_SIZE")

    def pick(d, pred):
        hits = [(k, v) for k, v in d.items() if pred(k)]
        if not hits:
            raise SystemExit("no kernel matched in the counter database")
        return hits[0][1]
    is_dom = lambda k: k.startswith("void " + kprefix) or k.startswith(kprefix)  # noqa: E731
    # the calibration copy moves COPY_BYTES in and COPY_BYTES out per launch; smaller copies of the
    # workload itself (an upload of routing offsets) are left out
    copy_f = _copy_calibration(fetch_db, "FETCH_SIZE")
    copy_w = _copy_calibration(write_db, "WRITE_SIZE")
    if workload == "moe":
        kf, nf = _grouped_gate_up_calls(fetch_db, "FETCH_SIZE")
        kw, nw = _grouped_gate_up_calls(write_db, "WRITE_SIZE")
    else:
        kf, nf = pick(fetch, is_dom)
        kw, nw = pick(write, is_dom)
    f_scale = COPY_BYTES / (copy_f * 1024.0)
    w_scale = COPY_BYTES / (copy_w * 1024.0)
    rec = {"kernel": kprefix, "workload": workload, "command": command,
           "source": os.path.relpath(src, ROOT), "source_sha256_16": src_hash(src),
           "fetch_kib_per_launch_raw": kf, "write_kib_per_launch_raw": kw, "launches": [nf, nw],
           "copy_fetch_kib_raw": copy_f, "copy_write_kib_raw": copy_w,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_fetch_bytes_per_launch": kf * 1024.0 * f_scale,
           "hbm_write_bytes_per_launch": kw * 1024.0 * w_scale}
    rec["hbm_bytes_per_launch"] = rec["hbm_fetch_bytes_per_launch"] + rec["hbm_write_bytes_per_launch"]
    out = out or os.path.join(ROOT, "profiles", fname)
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec))
    return rec


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense", choices=["dense", "recal", "decode", "moe", "train"])
    ap.add_argument("--mode", type=int, default=0, help="scale mode: 0 EXACT, 1 POW2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    ap.add_argument("--pmc-command", default="", help="the profiled command, recorded with --summarize-pmc")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.pmc_command)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(every kernel runs on one GPU's share at its real shape); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp8_x128_amd as fp8bs
    if not os.path.exists(fp8bs.LIB_PATH):
        from block_scaled_fp8_x128_amd import build
        build.build()
    fp8bs.lib()
    dev = torch.device("cuda", 0)
    timer = KernelTimer()
    common = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "data": "synthetic"}

    if args.workload == "dense":
        step, bufs, flops = dense_workload(fp8bs, dev, args.mode)
        ms = timed_loop(step, args.steps, args.warmup, timer)
        kernels, roof = summarize_dense(bufs, timer)
        out = {"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", **common,
               "ms_per_step": round(ms, 4), "dtype": "fp8e4m3",
               "config": {"workload": "8B-shaped dense layer at M=8192 tokens: recalibrate 4 weights (128x128, one batched launch), "
                                      "quantize 4 inputs (1x128), GEMMs QKV K4096 N6144, gate+up K4096 N28672, "
                                      "down K14336 N4096, o_proj K4096 N4096",
                          "scale_mode": "pow2" if args.mode else "exact", "out_dtype": "bf16",
                          "gemm_flops_per_step": flops},
               "roofline": roof, "kernels": kernels}
        cpu = (lambda: cpu_baseline_dense()) if not args.no_cpu_baseline else None
    elif args.workload == "train":
        step, bufs, flops = train_workload(fp8bs, dev, args.mode)
        ms = timed_loop(step, args.steps, args.warmup, timer)
        kernels, roof = summarize_train(bufs, timer)
        out = {"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", **common,
               "ms_per_step": round(ms, 4), "dtype": "fp8e4m3",
               "config": {"workload": "training backward of the 8B-shaped dense layer at M=8192 tokens: "
                                      "recalibrate 4 weights to W and W^T codes (one batched launch); per layer "
                                      "quantize dY along N and along the tokens (one read), data-gradient GEMM "
                                      "dX = dY W, quantize X^T along the tokens, weight-gradient GEMM dW = dY^T X; "
                                      "QKV, gate+up, down, o_proj",
                          "scale_mode": "pow2" if args.mode else "exact", "out_dtype": "bf16",
                          "gemm_flops_per_step": flops},
               "roofline": roof, "kernels": kernels}
        cpu = None
    elif args.workload == "recal":
        step, nbytes = recal_workload(fp8bs, dev)
        ms = timed_loop(step, args.steps, args.warmup, timer)
        te, tp = timer.avg_ms("recal_exact"), timer.avg_ms("recal_pow2")
        traffic, tsrc = traffic_for("recal")
        ach = nbytes / (te * 1e-3) / 1e9
        out = {"metric": METRIC, "value": round(2 * nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s", **common,
               "ms_per_step": round(ms, 4), "dtype": "bf16->fp8e4m3",
               "config": {"workload": "per-step recalibration: 32 layers x {6144x4096, 4096x4096, 28672x4096, "
                                      "4096x14336} bf16 weights, 128x128 blocks, EXACT then POW2",
                          "bytes_per_pass": nbytes},
               "roofline": {"kernel": DOMINANT["recal"][0] + " (batched, EXACT)", "bound": "hbm",
                            "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, "traffic_source": tsrc},
               "kernels": {"recal_exact": hbm_entry(te, nbytes), "recal_pow2": hbm_entry(tp, nbytes)}}
        cpu = (lambda: cpu_baseline_recal()) if not args.no_cpu_baseline else None
    elif args.workload == "decode":
        step, separate, pairs, flops = decode_workload(fp8bs, dev, args.mode)
        ms = timed_loop(step, args.steps, args.warmup, timer)
        separate(None, 2)
        separate(timer, args.steps)
        torch.cuda.synchronize()
        kernels = {}
        for p in pairs:
            tl = timer.avg_ms("linear_" + p["name"])
            tg = timer.avg_ms("gemm_" + p["name"])
            tq = timer.avg_ms("quant_" + p["name"])
            # GEMM alone: Wq + Ws + Xq + Xs + Y; the linear layer reads bf16 X instead of Xq + Xs
            wb = p["N"] * p["K"] * (1 + 4 / 16384) + p["M"] * p["N"] * 2
            gbytes = wb + p["M"] * p["K"] * (1 + 4 / 128)
            tf = lambda t, p=p: round(2.0 * p["M"] * p["N"] * p["K"] / (t * 1e-3) / 1e12, 2)
            kernels["linear_" + p["name"]] = {**hbm_entry(tl, wb + p["M"] * p["K"] * 2), "TFLOP/s": tf(tl),
                                              "fused": fp8bs.linear_workspace_size(p["M"], p["N"], p["K"]) == 0}
            kernels["gemm_" + p["name"]] = {**hbm_entry(tg, gbytes), "TFLOP/s": tf(tg)}
            kernels["quant_plus_gemm_" + p["name"]] = hbm_entry(tq + tg, gbytes + p["M"] * p["K"] * 2)
        # the step's longest single GEMM launch: the largest M (persistent kernel split along K)
        big = max(pairs, key=lambda p: p["N"] * p["K"] + p["M"])
        tb = timer.avg_ms("gemm_" + big["name"])
        nb = big["N"] * big["K"] * (1 + 4 / 16384) + big["M"] * big["K"] * (1 + 4 / 128) + big["M"] * big["N"] * 2
        ach = nb / (tb * 1e-3) / 1e9
        out = {"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", **common,
               "ms_per_step": round(ms, 4), "dtype": "fp8e4m3",
               "config": {"workload": "rollout decode: M in {1,16,64,256} x (gate+up K4096 N28672, down K14336 "
                                      "N4096), fp8_block_linear from bf16 activations (quantized inside the GEMM "
                                      "for M <= 16), 5 rotated weight copies"},
               "roofline": {"kernel": "fp8_block_gemm (persistent 128x256 kernel split along K), %s" % big["name"],
                            "bound": "hbm",
                            "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None},
               "kernels": kernels}
        cpu = None
    else:
        step, shapes, flops, E = moe_workload(fp8bs, dev, args.mode)
        ms = timed_loop(step, args.steps, args.warmup, timer)
        kernels = {}
        for name, (m, n, k) in shapes.items():
            t = timer.avg_ms("grouped_" + name)
            nbytes = m * k + m * k // 128 * 4 + E * n * k * (1 + 4 / 16384) + m * n * 2
            kernels["grouped_" + name] = {**mfma_entry(t, 2.0 * m * n * k), **hbm_entry(t, nbytes)}
        m, _, k = shapes["gate_up"]
        # dispatch quantizer: the token rows read once (T x K bf16), the row indices, codes and scales written
        kernels["quant_act_gather_gate_up"] = hbm_entry(timer.avg_ms("quant_act_gather_gate_up"),
                                                        T_TOKENS * k * 2 + m * 4 + m * k + m * k // 128 * 4)
        # gated activation + quantizer: 2 bf16 in, 1 code out per element of h, one fp32 per 128
        m, _, k = shapes["down"]
        kernels["swiglu_quant_down"] = hbm_entry(timer.avg_ms("swiglu_quant_down"), m * k * 5 + m * k // 128 * 4)
        t = timer.avg_ms("grouped_gate_up")
        m, n, k = shapes["gate_up"]
        # the roofline that binds: the gate+up call's algorithmic bytes at the HBM peak take longer
        # than its FLOPs at the FP8 peak (arithmetic intensity about 555 FLOP/B, below the ridge)
        gflop = 2.0 * m * n * k
        gbytes = m * k + m * k // 128 * 4 + E * n * k * (1 + 4 / 16384) + m * n * 2
        traffic, tsrc = traffic_for("moe")
        if gbytes / (PEAK_HBM_GBS * 1e9) >= gflop / (PEAK_FP8_TFLOPS * 1e12):
            ach = gbytes / (t * 1e-3) / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(ach / PEAK_HBM_GBS, 4)}
        else:
            ach = gflop / (t * 1e-3) / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / PEAK_FP8_TFLOPS, 4)}
        out = {"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", **common,
               "ms_per_step": round(ms, 4), "dtype": "fp8e4m3",
               "config": {"workload": "MoE layer: 128 experts, hidden 2048, expert FFN 768, 8192 tokens top-8 "
                                      "(65536 rows); the dispatch quantizing token rows into expert order, grouped "
                                      "gate+up K2048 N1536, the gated activation quantized for the down projection, "
                                      "grouped down K768 N2048"},
               "roofline": {"kernel": "fp8_block_grouped_gemm gate+up", **roof,
                            "algorithmic_bytes_per_launch": gbytes, "algorithmic_flop_per_launch": gflop,
                            "traffic": traffic, "traffic_source": tsrc},
               "kernels": kernels}
        cpu = None

    # median and min beside each per-kernel mean (entries keyed by their timer name)
    for k, v in out.get("kernels", {}).items():
        if isinstance(v, dict) and k in timer.pairs:
            med, mn = timer.spread(k)
            v["median_ms"], v["min_ms"] = round(med, 4), round(mn, 4)
    if args.copy_calibration:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev).view(torch.bfloat16)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if cpu is not None:
        log("timing the oracle on the host (bounded sample)")
        out["cpu_baseline"] = cpu()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
