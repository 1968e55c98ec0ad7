"""Benchmark of the block-FP8 linear-layer hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input.
Workloads (--workload):
  all    (default) the dense layer below in EXACT mode is the headline (value,
         roofline, cpu_baseline); then every other measured row, each with its
         own roofline object and oracle CPU baseline (all threads and one):
         d1 the 32-layer recalibration (EXACT, POW2), d2 the activation
         quantizer alone at its four shapes beside a device copy of the same
         bytes, d3 the dense layer with power-of-2 scales, d4 the decode grid,
         d5 the MoE layer (EXACT, POW2), d6 the tiny layer's latency, the
         GEMM that quantizes its own output against GEMM + quantizer, and
         the decode attention over an FP8 KV cache.
  dense  8B-shaped dense layer at M = 8192 tokens: per-step
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
         routed top-8: expert-weight recalibration, the dispatch (each token
         row quantized once and written to its 8 expert rows), the grouped
         gate+up GEMM, the gated activation quantized for the down input, the
         grouped down GEMM.
Prints ONE JSON line.  `value` is GEMM TFLOP/s over the whole step
(quantizers included) except for `recal` (GB/s).  Per-kernel times come from
HIP events recorded on the stream the library launches on (torch's current
stream, whose handle every call passes to the library).

Tool modes (no GPU work of their own):
  --copy-calibration   after the timed steps, copy a 1 GiB buffer three times
                       (a plain copy kernel of known size, the reference for
                       scaling rocprofv3 FETCH_SIZE / WRITE_SIZE);
  --summarize-trace TRACE_DB OUT_MD  summarize a rocprofv3 --kernel-trace
                       database of the default run (per-kernel statistics and
                       the headline kernel's timed dispatches);
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
    "dense": ("fp8bs::gemm_dma_kernel<256, 256, 4, 2, false, false, false, false, false, 0>", GEMM_SRC,
              "gemm_dma_256x256_dense_m8192_traffic.json"),
    "recal": ("fp8bs::quant_w_kernel<0, 4>", QUANT_SRC, "quant_w_recal_32layers_traffic.json"),
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

def dense_data(dev):
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
    return bufs


def dense_step(fp8bs, bufs, mode):
    # POW2 scales go to the entry points that apply them through the matrix cores
    gemm = fp8bs.fp8_block_gemm_pow2 if mode else fp8bs.fp8_block_gemm
    w_all = [b["w"] for b in bufs]
    out_all = [(b["wq"], b["ws"]) for b in bufs]

    def step(timer):
        # the step's recalibration: all four weights in one batched launch
        maybe(timer, "quant_w_all", lambda: fp8bs.quant_w_128x128_batched(w_all, mode, outs=out_all))
        for b in bufs:
            maybe(timer, "quant_act_" + b["name"], lambda: fp8bs.quant_act_1x128(b["x"], mode, out=(b["xq"], b["xs"])))
            maybe(timer, "gemm_" + b["name"],
                  lambda: gemm(b["xq"], b["xs"], b["wq"], b["ws"], out=b["y"]))

    return step


def dense_workload(fp8bs, dev, mode):
    bufs = dense_data(dev)
    flops = sum(2.0 * b["M"] * b["N"] * b["K"] for b in bufs)
    return dense_step(fp8bs, bufs, mode), bufs, flops


def train_workload(fp8bs, dev, mode):
    """Backward data gradients of the same four layers: dX [M, K] = dY [M, N] W [N, K]."""
    gemm = fp8bs.fp8_block_gemm_pow2 if mode else fp8bs.fp8_block_gemm
    wgrad = fp8bs.fp8_block_gemm_1x128_pow2 if mode else fp8bs.fp8_block_gemm_1x128
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
                  lambda: wgrad(b["dyt"][0], b["dyt"][1], b["xt"][0], b["xt"][1], out=b["dw"]))

    # data and weight gradients: twice the forward FLOPs
    flops = sum(4.0 * b["M"] * b["N"] * b["K"] for b in bufs)
    return step, bufs, flops


def summarize_train(bufs, timer, mode=0):
    """The data-gradient half as summarize_dense, plus the weight-gradient GEMMs and
    the transposing quantizers; the roofline object covers whichever GEMM kernel
    takes more of the step (with POW2 scales: the kernels that take them on the
    matrix cores)."""
    kernels, roof = summarize_dense(bufs, timer, dual=True)
    if mode:
        roof["kernel"] = roof["kernel"].replace("false, false, false, false, false, 0>",
                                                "false, false, false, true, false, 0>")
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
        roof = {"kernel": "fp8bs::gemm_dma_kernel<256, 256, 4, 2, false, false, false, %s, true, 0> (weight "
                          "gradients of QKV, gate+up, down, o_proj over 8192 tokens)" % ("true" if mode else "false"),
                "bound": "mfma",
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
            wq, ws = fp8bs.quant_w_128x128(synth.weights_dev(N, K, dev, sub=synth.sub_layer(40 + c)), mode)
            copies.append((wq, ws))
        for j, M in enumerate((1, 16, 64, 256)):
            x = synth.activations_dev(M, K, dev, sub=synth.SUB_X + M)
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

    def stream(timer, reps):
        # five back-to-back calls of one pair per event pair, one per weight copy (each copy last read
        # four calls, 235 MB or more of weights, earlier): the per-launch time without each launch's
        # own start-up, as in a decode step that runs its layers back to back
        for r in range(reps):
            for p in pairs:
                def gemms(p=p):
                    for c in range(5):
                        wq, ws = p["copies"][(r + p["j"] + 1 + c) % 5]
                        gemm(p["xq"], p["xs"], wq, ws, out=p["y"], workspace=p["ws_buf"])

                def linears(p=p):
                    for c in range(5):
                        wq, ws = p["copies"][(r + p["j"] + 1 + c) % 5]
                        linear(p["x"], wq, ws, out=p["y"], workspace=p["lin_buf"])
                maybe(timer, "gemm5_" + p["name"], gemms)
                maybe(timer, "linear5_" + p["name"], linears)

    step.stream = stream
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
    # the dispatch: each token row is read and quantized once and written to its 8 expert rows
    # (the gather form, timed beside the step, reads each token row once per routed copy)
    xt = synth.activations_dev(T, H, dev, sub=synth.SUB_X)
    rows_d = torch.from_numpy(np.ascontiguousarray(row_token, dtype=np.int32)).to(dev)
    dest_d = torch.from_numpy(synth.moe_dest(row_token, T, TOPK)).to(dev)
    w1 = synth.weights_dev(E * 2 * F, H, dev, sub=synth.SUB_W)
    w2 = synth.weights_dev(E * H, F, dev, sub=synth.SUB_W + 1)
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
        maybe(timer, "quant_act_scatter_gate_up", lambda: fp8bs.quant_act_1x128_scatter(xt, dest_d, Mt, mode,
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

    def gather_form(timer, reps):
        # the gather form of the same dispatch (same outputs), timed after the steps for comparison
        for _ in range(reps):
            maybe(timer, "quant_act_gather_gate_up", lambda: fp8bs.quant_act_1x128_gather(xt, rows_d, mode,
                                                                                        out=(b["x1q"], b["x1s"])))
    step.gather_form = gather_form
    return step, shapes, flops, E


# ---------------------------------------------------------------------------
# the default run: every measured row of the hot path
# ---------------------------------------------------------------------------

CPU_TARGET_S = 2.5  # wall time per oracle sample and thread count (all threads, then one)
ACT_BPE = 3.0 + 4.0 / 128      # activation quantizer: bf16 in, code out, one fp32 per 128
W_BPE = 3.0 + 4.0 / 16384      # weight quantizer: the same with one fp32 per 128 x 128


def cpu_row(make, work_of, unit, describe, n0, nmax, target_s=CPU_TARGET_S):
    """The oracle on a bounded sample: make(n) prepares a sample of size n
    (outside the clock) and returns (callable, n actually used); the sample
    grows until one call takes target_s, once with all of the oracle's threads
    and once with one.  value = work_of(n) / seconds."""
    import oracle
    allt = oracle.max_threads()
    res = {}
    for th in (allt, 1):
        oracle.set_threads(th)
        n = n0
        while True:
            f, n_used = make(n)
            t0 = time.perf_counter()
            f()
            dt = time.perf_counter() - t0
            if dt >= target_s or n_used >= nmax:
                break
            n = min(nmax, max(n * 2, int(n * target_s / max(dt, 1e-3) * 1.1)))
        res[th] = (n_used, dt)
    oracle.set_threads(allt)
    (n, dt), (n1, dt1) = res[allt], res[1]
    return {"value": work_of(n) / dt, "unit": unit, "cores": allt, "kind": "oracle",
            "sample": describe(n, dt), "value_1thread": work_of(n1) / dt1, "sample_1thread": describe(n1, dt1)}


def roof_hbm(kernel, ms, nbytes, traffic=None, tsrc=None):
    ach = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic, "traffic_source": tsrc,
            "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": round(ms, 4)}


def roof_mfma(kernel, ms, flops, traffic=None, tsrc=None):
    ach = flops / (ms * 1e-3) / 1e12
    return {"kernel": kernel, "bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": traffic, "traffic_source": tsrc,
            "algorithmic_flop_per_launch": flops, "avg_launch_ms": round(ms, 4)}


def roof_binding(kernel, ms, flops, nbytes, traffic=None, tsrc=None):
    """The roofline that binds: HBM when the algorithmic bytes at the HBM peak take
    longer than the FLOPs at the FP8 peak, else the matrix cores."""
    if nbytes / (PEAK_HBM_GBS * 1e9) >= flops / (PEAK_FP8_TFLOPS * 1e12):
        r = roof_hbm(kernel, ms, nbytes, traffic, tsrc)
        r["algorithmic_flop_per_launch"] = flops
    else:
        r = roof_mfma(kernel, ms, flops, traffic, tsrc)
        r["algorithmic_bytes_per_launch"] = nbytes
    return r


def with_spread(kernels, timer):
    for k, v in kernels.items():
        if isinstance(v, dict) and k in timer.pairs:
            med, mn = timer.spread(k)
            v["median_ms"], v["min_ms"] = round(med, 4), round(mn, 4)
    return kernels


def cpu_recal(target_s=CPU_TARGET_S):
    """d1: the oracle's 128x128 quantizer on the first rows of a 28672 x 4096 weight."""
    import oracle
    import synth
    w = synth.weights(28672, 4096, sub=synth.sub_layer(0))

    def make(n):
        r = max(128, min(28672, n // (128 * 4096) * 128))
        wr = np.ascontiguousarray(w[:r])
        return (lambda: oracle.quant_w_128x128(wr, 0)), r * 4096
    return cpu_row(make, lambda n: n * W_BPE / 1e9, "GB/s",
                   lambda n, dt: "quant_w_128x128 (EXACT) of the first %d rows of one 28672 x 4096 weight, %.2f s "
                                 "wall" % (n // 4096, dt), 1 << 21, 28672 * 4096, target_s)


def cpu_quant_act(target_s=CPU_TARGET_S):
    """d2: the oracle's 1x128 quantizer on the first rows of X [8192, 4096]."""
    import oracle
    import synth
    x = synth.activations(8192, 4096, sub=synth.SUB_X)

    def make(n):
        r = max(1, min(8192, n // 4096))
        xr = np.ascontiguousarray(x[:r])
        return (lambda: oracle.quant_act_1x128(xr, 0)), r * 4096
    return cpu_row(make, lambda n: n * ACT_BPE / 1e9, "GB/s",
                   lambda n, dt: "quant_act_1x128 (EXACT) of the first %d rows of X [8192, 4096], %.2f s wall"
                                 % (n // 4096, dt), 1 << 20, 8192 * 4096, target_s)


def cpu_decode(target_s=CPU_TARGET_S):
    """d4: the oracle's linear layer (quant_act_1x128 + gemm_full) at M = 16 against the gate+up weight."""
    import oracle
    import synth
    N, K = 28672, 4096
    w = synth.weights(N, K, sub=synth.sub_layer(40))
    wq, ws = oracle.quant_w_128x128(w)
    x = synth.activations(16, K, sub=synth.SUB_X + 16)

    def make(n):
        reps = max(1, n)

        def f():
            for _ in range(reps):
                xq, xs = oracle.quant_act_1x128(x)
                oracle.gemm_full(xq, xs, wq, ws)
        return f, reps
    lb = N * K * (1 + 4 / 16384) + 16 * N * 2 + 16 * K * 2
    return cpu_row(make, lambda r: r * lb / 1e9, "GB/s",
                   lambda r, dt: "%d oracle linear layers (quant_act_1x128 + gemm_full) at M = 16 against the "
                                 "gate+up weight, %.2f s wall" % (r, dt), 1, 64, target_s)


def cpu_moe(target_s=CPU_TARGET_S, experts=16):
    """d5: the oracle's full-output grouped GEMM (gate+up) over the first experts' routed rows."""
    import oracle
    import synth
    row_token, offs = synth.moe_routing(T_TOKENS, 128, 8)
    N, K = 1536, 2048
    x_tok = synth.activations(T_TOKENS, K, sub=synth.SUB_X)
    w = synth.weights(experts * N, K, sub=synth.SUB_W)
    wq, ws = oracle.quant_w_128x128(w)
    wq, ws = wq.reshape(experts, N, K), ws.reshape(experts, N // 128, K // 128)

    def make(n):
        e = max(1, min(experts, n))
        xq, xs = oracle.quant_act_1x128(np.ascontiguousarray(x_tok[row_token[:int(offs[e])]]))
        return (lambda: oracle.grouped_gemm_full(xq, xs, wq[:e], ws[:e], offs[:e + 1])), e
    return cpu_row(make, lambda e: 2.0 * int(offs[e]) * N * K / 1e12, "TFLOP/s",
                   lambda e, dt: "grouped_gemm_full (every output) of the gate+up GEMM over the first %d of 128 "
                                 "experts (%d rows), %.2f s wall" % (e, int(offs[e]), dt), 1, experts, target_s)


def cpu_tiny(target_s=CPU_TARGET_S):
    """d6: the oracle's whole tiny layer (quant_act_1x128 + quant_w_128x128 + gemm_full), repeated."""
    import oracle
    import synth
    xh, wh = synth.activations(256, 512), synth.weights(512, 512)

    def make(n):
        reps = max(1, n)

        def f():
            for _ in range(reps):
                a, b = oracle.quant_act_1x128(xh)
                c, d = oracle.quant_w_128x128(wh)
                oracle.gemm_full(a, b, c, d)
        return f, reps
    cb = cpu_row(make, lambda r: r, "layers/s",
                 lambda r, dt: "%d oracle tiny layers (quant_act_1x128 + quant_w_128x128 + gemm_full), %.2f s wall"
                               % (r, dt), 1, 1 << 16, target_s)
    cb["latency_ms"] = round(1e3 / cb["value"], 3)
    cb["latency_ms_1thread"] = round(1e3 / cb["value_1thread"], 3)
    return cb


def row_recal(fp8bs, dev, steps, warmup, cpu):
    """d1: 32 layers x 4 weights re-quantized, EXACT then POW2."""
    timer = KernelTimer()
    step, nbytes = recal_workload(fp8bs, dev)
    ms = timed_loop(step, steps, warmup, timer)
    traffic, tsrc = traffic_for("recal")
    out = {"config": "32 layers x {6144x4096, 4096x4096, 28672x4096, 4096x14336} bf16 weights, 128x128 blocks, "
                     "one quant_w_128x128_batched call per mode (32 tensors per launch)",
           "ms_per_step": round(ms, 4), "bytes_per_pass": nbytes}
    for mode, name in ((0, "exact"), (1, "pow2")):
        t = timer.avg_ms("recal_" + name)
        out[name] = {**hbm_entry(t, nbytes), "roofline": roof_hbm(DOMINANT["recal"][0].replace("<0,", "<%d," % mode)
                                                                  + " (batched)", t, nbytes,
                                                                  *((traffic, tsrc) if mode == 0 else (None, None)))}
    with_spread({"recal_exact": out["exact"], "recal_pow2": out["pow2"]}, timer)
    if cpu:
        out["cpu_baseline"] = cpu_recal()
    return out


def row_quant_act(fp8bs, dev, steps, warmup, cpu):
    """d2: the activation quantizer alone at the four activation shapes, each
    beside the runtime's device copy of the same byte count (half read, half
    written).  Timed two ways:
    - single: one launch between two events, after a 512 MiB read that keeps
      the input out of the 256 MB infinity cache (a write there would leave
      dirty lines whose write-back the next launch would pay for); the events
      also count the launch's own start-up;
    - stream (the roofline figure): R back-to-back launches between two
      events, each on its own input and output copy, R copies holding more
      than 600 MB, so that every launch reads an input last touched more than
      500 MB of traffic earlier (out of the cache) and the launches' start-up
      overlaps the previous launch, as in a layer step."""
    import synth
    import torch
    shapes = [(8192, 4096), (8192, 14336), (65536, 2048), (65536, 768)]
    scrub = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    out = {"config": "quant_act_1x128 (EXACT) alone on [8192,4096] and [8192,14336] (8B dense layer inputs) and "
                     "[65536,2048] and [65536,768] (MoE gate+up and down inputs); cold inputs; stream = R "
                     "back-to-back launches on R rotated input/output copies (> 600 MB) per event pair, single = "
                     "one launch per event pair after a cache-evicting read; copy = torch copy_ of a uint8 "
                     "buffer of half the algorithmic bytes, timed the same two ways"}
    timer = KernelTimer()
    for i, (M, K) in enumerate(shapes):
        nbytes = M * K * ACT_BPE
        R = max(2, int(-(-600e6 // nbytes)))
        x0 = synth.activations_dev(M, K, dev, sub=synth.SUB_X + 50 + i)
        xs_in = [x0] + [x0.clone() for _ in range(R - 1)]
        outs = [(torch.empty((M, K), dtype=torch.uint8, device=dev),
                 torch.empty((M, K // 128), dtype=torch.float32, device=dev)) for _ in range(R)]
        half = int(nbytes // 2) // 16 * 16
        srcs = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(R)]
        dsts = [torch.empty(half, dtype=torch.uint8, device=dev) for _ in range(R)]
        name = "%dx%d" % (M, K)

        # (copies 1 .. R - 1, then 0: the single launch just read copy 0)
        order = list(range(1, R)) + [0]

        def quant_burst():
            for c in order:
                fp8bs.quant_act_1x128(xs_in[c], 0, out=outs[c])

        def copy_burst():
            for c in order:
                dsts[c].copy_(srcs[c])
        for r in range(warmup + steps):
            t = timer if r >= warmup else None
            scrub.max()
            maybe(t, "quant1_" + name, lambda: fp8bs.quant_act_1x128(xs_in[0], 0, out=outs[0]))
            scrub.max()
            maybe(t, "copy1_" + name, lambda: dsts[0].copy_(srcs[0]))
            maybe(t, "quantR_" + name, quant_burst)
            maybe(t, "copyR_" + name, copy_burst)
        torch.cuda.synchronize()
        tq, tc = timer.avg_ms("quantR_" + name) / R, timer.avg_ms("copyR_" + name) / R
        t1q, t1c = timer.avg_ms("quant1_" + name), timer.avg_ms("copy1_" + name)
        med, mn = timer.spread("quantR_" + name)
        out[name] = {**hbm_entry(tq, nbytes), "median_ms": round(med / R, 4), "min_ms": round(mn / R, 4),
                     "copies": R, "copy_ms": round(tc, 4), "copy_GB/s": round(2 * half / (tc * 1e-3) / 1e9, 1),
                     "frac_of_copy": round(tc / tq, 4),
                     "single": {**hbm_entry(t1q, nbytes), "copy_ms": round(t1c, 4)},
                     "roofline": roof_hbm("fp8bs::quant_act_kernel", tq, nbytes)}
        del x0, xs_in, outs, srcs, dsts
        torch.cuda.empty_cache()
    del scrub
    torch.cuda.empty_cache()
    if cpu:
        out["cpu_baseline"] = cpu_quant_act()
    return out


def row_dense_pow2(fp8bs, bufs, steps, warmup):
    """d3 with power-of-2 scales: the same layer through the _pow2 entry points."""
    timer = KernelTimer()
    ms = timed_loop(dense_step(fp8bs, bufs, 1), steps, warmup, timer)
    kernels, roof = summarize_dense(bufs, timer)
    roof["kernel"] = roof["kernel"].replace("false, false, false, false, false, 0>", "false, false, false, true, false, 0>")
    roof["traffic"], roof["traffic_source"] = None, None
    flops = sum(2.0 * b["M"] * b["N"] * b["K"] for b in bufs)
    return {"ms_per_step": round(ms, 4), "TFLOP/s_step": round(flops / (ms * 1e-3) / 1e12, 2),
            "roofline": roof, "kernels": with_spread(kernels, timer)}


def cpu_dense(target_s=CPU_TARGET_S):
    """d3: the oracle's full-output GEMM on the first rows of the gate+up GEMM."""
    import oracle
    import synth
    N, K = 28672, 4096
    w = synth.weights(N, K, sub=synth.sub_layer(1))
    wq, ws = oracle.quant_w_128x128(w)
    x = synth.activations(1024, K, sub=synth.SUB_X + 10)
    xq, xs = oracle.quant_act_1x128(x)

    def make(n):
        r = max(1, min(1024, n))
        a, b = np.ascontiguousarray(xq[:r]), np.ascontiguousarray(xs[:r])
        return (lambda: oracle.gemm_full(a, b, wq, ws)), r
    return cpu_row(make, lambda r: 2.0 * r * N * K / 1e12, "TFLOP/s",
                   lambda r, dt: "gemm_full (every output) of the gate+up GEMM (N 28672, K 4096), first %d of 8192 "
                                 "rows, %.2f s wall" % (r, dt), 8, 1024, target_s)


def row_decode(fp8bs, dev, steps, warmup, cpu):
    """d4: M in {1, 16, 64, 256} against the gate+up and down weights, through
    fp8_block_linear, and the GEMM alone beside it; 5 rotated weight copies."""
    timer = KernelTimer()
    step, separate, pairs, flops = decode_workload(fp8bs, dev, 0)
    ms = timed_loop(step, steps, warmup, timer)
    separate(None, 2)
    separate(timer, steps)
    step.stream(None, 1)
    step.stream(timer, steps)
    import torch
    torch.cuda.synchronize()
    out = {"config": "M in {1,16,64,256} x (gate+up K4096 N28672, down K14336 N4096), EXACT; linear = "
                     "fp8_block_linear from bf16 X (one launch for M <= 16), gemm = fp8_block_gemm alone; "
                     "per call: one call per event pair (its own start-up included); roofline: five calls "
                     "back to back per event pair, one per rotated weight copy",
           "ms_per_step": round(ms, 4)}
    for p in pairs:
        tl, tg = timer.avg_ms("linear_" + p["name"]), timer.avg_ms("gemm_" + p["name"])
        tl5, tg5 = timer.avg_ms("linear5_" + p["name"]) / 5, timer.avg_ms("gemm5_" + p["name"]) / 5
        wb = p["N"] * p["K"] * (1 + 4 / 16384) + p["M"] * p["N"] * 2
        gbytes = wb + p["M"] * p["K"] * (1 + 4 / 128)
        lbytes = wb + p["M"] * p["K"] * 2
        fl = 2.0 * p["M"] * p["N"] * p["K"]
        lm, lmin = timer.spread("linear_" + p["name"])
        gm, gmin = timer.spread("gemm_" + p["name"])
        out[p["name"]] = {
            "linear": {**hbm_entry(tl5, lbytes), "per_call_ms": round(tl, 4), "per_call_median_ms": round(lm, 4),
                       "per_call_min_ms": round(lmin, 4),
                       "fused": fp8bs.linear_workspace_size(p["M"], p["N"], p["K"]) == 0,
                       "roofline": roof_hbm("fp8_block_linear", tl5, lbytes)},
            "gemm": {**hbm_entry(tg5, gbytes), "per_call_ms": round(tg, 4), "per_call_median_ms": round(gm, 4),
                     "per_call_min_ms": round(gmin, 4),
                     "roofline": roof_binding("fp8_block_gemm", tg5, fl, gbytes)}}
    del pairs
    torch.cuda.empty_cache()
    if cpu:
        out["cpu_baseline"] = cpu_decode()
    return out


def row_moe(fp8bs, dev, steps, warmup, cpu):
    """d5: the MoE layer, EXACT then POW2."""
    import torch
    out = {"config": "128 experts, hidden 2048, expert FFN 768, 8192 tokens top-8 (65536 rows): dispatch quantizer, "
                     "grouped gate+up K2048 N1536, gated activation + quantizer, grouped down K768 N2048"}
    for mode, mname in ((0, "exact"), (1, "pow2")):
        timer = KernelTimer()
        step, shapes, flops, E = moe_workload(fp8bs, dev, mode)
        ms = timed_loop(step, steps, warmup, timer)
        step.gather_form(None, 2)
        step.gather_form(timer, steps)
        torch.cuda.synchronize()
        r = {"ms_per_step": round(ms, 4), "TFLOP/s_step": round(flops / (ms * 1e-3) / 1e12, 2)}
        traffic, tsrc = traffic_for("moe") if mode == 0 else (None, None)
        for name, (m, n, k) in shapes.items():
            t = timer.avg_ms("grouped_" + name)
            nbytes = m * k + m * k // 128 * 4 + E * n * k * (1 + 4 / 16384) + m * n * 2
            fl = 2.0 * m * n * k
            med, mn = timer.spread("grouped_" + name)
            tr = (traffic, tsrc) if name == "gate_up" else (None, None)
            r["grouped_" + name] = {"ms": round(t, 4), "median_ms": round(med, 4), "min_ms": round(mn, 4),
                                    "roofline": roof_binding("fp8_block_grouped_gemm%s %s" %
                                                             ("_pow2" if mode else "", name), t, fl, nbytes, *tr)}
        m, _, k = shapes["gate_up"]
        for dname in ("quant_act_scatter_gate_up", "quant_act_gather_gate_up"):
            r[dname] = hbm_entry(timer.avg_ms(dname), T_TOKENS * k * 2 + m * 4 + m * k + m * k // 128 * 4)
        m, _, k = shapes["down"]
        r["swiglu_quant_down"] = hbm_entry(timer.avg_ms("swiglu_quant_down"), m * k * 5 + m * k // 128 * 4)
        r["quant_w_experts"] = hbm_entry(timer.avg_ms("quant_w_experts"),
                                         E * (2 * 768 * 2048 + 2048 * 768) * W_BPE)
        out[mname] = r
        del step
        torch.cuda.empty_cache()
    if cpu:
        out["cpu_baseline"] = cpu_moe()
    return out


def row_tiny(fp8bs, dev, steps, warmup, cpu):
    """d6: the tiny linear layer (X [256, 512], W [512, 512], seed 0): latency of
    quant_act_1x128 + quant_w_128x128 + fp8_block_gemm, reported, not rooflined."""
    import synth
    import torch
    M, N, K = 256, 512, 512
    x = bf16_dev(synth.activations(M, K), dev)
    w = bf16_dev(synth.weights(N, K), dev)
    xq, xs = torch.empty((M, K), dtype=torch.uint8, device=dev), torch.empty((M, K // 128), dtype=torch.float32,
                                                                              device=dev)
    wq, ws = torch.empty((N, K), dtype=torch.uint8, device=dev), torch.empty((N // 128, K // 128),
                                                                              dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    timer = KernelTimer()
    reps = max(100, 5 * steps)
    for r in range(warmup + reps):
        t = timer if r >= warmup else None

        def layer():
            fp8bs.quant_act_1x128(x, 0, out=(xq, xs))
            fp8bs.quant_w_128x128(w, 0, out=(wq, ws))
            fp8bs.fp8_block_gemm(xq, xs, wq, ws, out=y)
        maybe(t, "layer", layer)
        maybe(t, "gemm", lambda: fp8bs.fp8_block_gemm(xq, xs, wq, ws, out=y))
    torch.cuda.synchronize()
    # the same three calls captured once in a HIP graph and replayed: one launch per layer, no
    # per-call host work (the library issues kernel launches only, so the calls capture as they are)
    def layer():
        fp8bs.quant_act_1x128(x, 0, out=(xq, xs))
        fp8bs.quant_w_128x128(w, 0, out=(wq, ws))
        fp8bs.fp8_block_gemm(xq, xs, wq, ws, out=y)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        layer()
    torch.cuda.synchronize()
    for r in range(warmup + reps):
        maybe(timer if r >= warmup else None, "layer_graph", graph.replay)
    torch.cuda.synchronize()
    lm, lmin = timer.spread("layer")
    gm, gmin = timer.spread("gemm")
    grm, grmin = timer.spread("layer_graph")
    out = {"config": "X [256,512], W [512,512], seed 0, EXACT: quant_act_1x128 + quant_w_128x128 + fp8_block_gemm "
                     "(bf16 out), three launches on one stream, %d timed repetitions; layer_graph: the three "
                     "calls captured in one HIP graph, one replay per event pair" % reps,
           "latency_us": {"layer_median": round(lm * 1e3, 2), "layer_min": round(lmin * 1e3, 2),
                          "gemm_median": round(gm * 1e3, 2), "gemm_min": round(gmin * 1e3, 2),
                          "layer_graph_median": round(grm * 1e3, 2), "layer_graph_min": round(grmin * 1e3, 2)},
           "flops": 2.0 * M * N * K}
    if cpu:
        out["cpu_baseline"] = cpu_tiny()
    return out


def row_gemm_quant(fp8bs, dev, steps, warmup, cpu):
    """NEXT-2: a GEMM whose output feeds another FP8 GEMM, at the o_proj and QKV shapes (M = 8192):
    fp8_block_gemm then quant_act_1x128 of its bf16 output, against fp8_block_gemm_quant (codes and
    scales from the GEMM's epilogue), with and without the bf16 output."""
    import synth
    import torch
    out = {"config": "M=8192, EXACT: 'separate' = fp8_block_gemm (bf16 Y) + quant_act_1x128(Y); 'fused' = "
                     "fp8_block_gemm_quant with Y; 'fused_codes_only' = fp8_block_gemm_quant without Y"}
    for name, N, K in (("o_proj", 4096, 4096), ("qkv", 6144, 4096)):
        M = 8192
        xq, xs = fp8bs.quant_act_1x128(synth.activations_dev(M, K, dev, sub=synth.SUB_X + 80))
        wq, ws = fp8bs.quant_w_128x128(synth.weights_dev(N, K, dev, sub=synth.sub_layer(80)))
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        yq = torch.empty((M, N), dtype=torch.uint8, device=dev)
        ys = torch.empty((M, N // 128), dtype=torch.float32, device=dev)
        timer = KernelTimer()

        def sep():
            fp8bs.fp8_block_gemm(xq, xs, wq, ws, out=y)
            fp8bs.quant_act_1x128(y, 0, out=(yq, ys))
        for r in range(warmup + steps):
            t = timer if r >= warmup else None
            maybe(t, "separate", sep)
            maybe(t, "fused", lambda: fp8bs.fp8_block_gemm_quant(xq, xs, wq, ws, 0, out=(y, yq, ys)))
            maybe(t, "fused_codes_only", lambda: fp8bs.fp8_block_gemm_quant(xq, xs, wq, ws, 0, out=(None, yq, ys)))
        torch.cuda.synchronize()
        fl = 2.0 * M * N * K
        out[name] = {k: {**mfma_entry(timer.avg_ms(k), fl), "median_ms": round(timer.spread(k)[0], 4)}
                     for k in ("separate", "fused", "fused_codes_only")}
        out[name]["fused_saving_frac"] = round(1 - timer.avg_ms("fused") / timer.avg_ms("separate"), 4)
        del xq, xs, wq, ws, y, yq, ys
    torch.cuda.empty_cache()
    return out


ATT = dict(B=64, T=4096, Hq=32, Hkv=8)  # decode attention: 64 sequences, 4096 cached tokens, Llama-3.1-8B heads


def cpu_attention(target_s=CPU_TARGET_S):
    """The oracle's fp64 attention over the FP8 cache: sequences of 4096 tokens, 32 / 8 heads."""
    import oracle
    import synth
    T, Hq, Hkv = ATT["T"], ATT["Hq"], ATT["Hkv"]
    k = synth.activations(T, Hkv * 128, sub=synth.SUB_X)
    v = synth.activations(T, Hkv * 128, sub=synth.SUB_W)
    kq, ks = oracle.quant_act_1x128(k)
    vq, vs = oracle.quant_act_1x128(v)
    q1 = synth.activations(Hq, 128, sub=synth.SUB_DY)

    def make(n):
        b = max(1, min(64, n))
        shape = (b, T, Hkv)
        kq_b = np.ascontiguousarray(np.broadcast_to(kq.reshape(1, T, Hkv, 128), shape + (128,)))
        vq_b = np.ascontiguousarray(np.broadcast_to(vq.reshape(1, T, Hkv, 128), shape + (128,)))
        ks_b = np.ascontiguousarray(np.broadcast_to(ks.reshape(1, T, Hkv), shape))
        vs_b = np.ascontiguousarray(np.broadcast_to(vs.reshape(1, T, Hkv), shape))
        q = np.ascontiguousarray(np.broadcast_to(q1.reshape(1, Hq, 128), (b, Hq, 128)))
        lens = np.full(b, T, np.int32)
        return (lambda: oracle.kv_attention_decode(q, kq_b, ks_b, vq_b, vs_b, lens, 0.088388)), b
    per_seq = T * Hkv * 2 * (128 + 4)
    return cpu_row(make, lambda b: b * per_seq / 1e9, "GB/s",
                   lambda b, dt: "kv_attention_decode of %d sequences x %d cached tokens (32 query / 8 key-value "
                                 "heads), %.2f s wall" % (b, T, dt), 1, 64, target_s)


def row_attention(fp8bs, dev, steps, warmup, cpu):
    """NEXT-4: decode attention over the FP8 KV cache, one layer: 64 sequences x 4096 cached
    tokens, 32 query / 8 key-value heads of dim 128; the cache written by quant_act_1x128."""
    import synth
    import torch
    B, T, Hq, Hkv = ATT["B"], ATT["T"], ATT["Hq"], ATT["Hkv"]
    k = synth.activations_dev(B * T, Hkv * 128, dev, sub=synth.SUB_X + 70)
    v = synth.activations_dev(B * T, Hkv * 128, dev, sub=synth.SUB_W + 70)
    kq, ks = fp8bs.quant_act_1x128(k)
    vq, vs = fp8bs.quant_act_1x128(v)
    del k, v
    kq, vq = kq.view(B, T, Hkv, 128), vq.view(B, T, Hkv, 128)
    ks, vs = ks.view(B, T, Hkv), vs.view(B, T, Hkv)
    q = synth.activations_dev(B * Hq, 128, dev, sub=synth.SUB_DY + 70).view(B, Hq, 128)
    lens = torch.full((B,), T, dtype=torch.int32, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(max(1, fp8bs.kv_attention_workspace_size(B, T, Hq, Hkv)), dtype=torch.uint8, device=dev)
    scrub = torch.zeros(512 << 20, dtype=torch.uint8, device=dev)
    timer = KernelTimer()
    for r in range(warmup + steps):
        t = timer if r >= warmup else None
        scrub.max()   # (the 554 MB cache is larger than the 256 MB infinity cache anyway)
        maybe(t, "attn", lambda: fp8bs.fp8_kv_attention_decode(q, kq, ks, vq, vs, lens, 0.088388, out=out,
                                                                workspace=ws))
    torch.cuda.synchronize()
    ta = timer.avg_ms("attn")
    med, mn = timer.spread("attn")
    nbytes = 2 * B * T * Hkv * (128 + 4) + B * Hq * 128 * 2 * 2 + B * 4
    out_d = {"config": "one layer: %d sequences x %d cached tokens, %d query / %d key-value heads of dim 128, "
                       "E4M3 cache with one fp32 scale per token and head, bf16 out" % (B, T, Hq, Hkv),
             "attention": {**hbm_entry(ta, nbytes), "median_ms": round(med, 4), "min_ms": round(mn, 4),
                           "splits_workspace_bytes": fp8bs.kv_attention_workspace_size(B, T, Hq, Hkv),
                           "roofline": roof_hbm("fp8bs::kv_attn_decode_kernel<4>", ta, nbytes)},
             "bf16_cache_roofline_ms": round((nbytes + 2 * B * T * Hkv * 124) / (PEAK_HBM_GBS * 1e9) * 1e3, 4)}
    del kq, vq, ks, vs, scrub
    torch.cuda.empty_cache()
    if cpu:
        out_d["cpu_baseline"] = cpu_attention()
    return out_d


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
            after_quant = any(q in k for q in ("quant_act_kernel", "quant_act_gather_kernel",
                                               "quant_act_scatter_kernel"))
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


def summarize_trace(db, command, steps, warmup, out, workload="all"):
    """Markdown summary of a rocprofv3 --kernel-trace database of `bench.py --workload
    workload`: per kernel the dispatch count and duration statistics and, for the default run
    and the dense workload, the headline kernel's timed dispatches (the dense layer's four
    GEMMs of steps warmup .. warmup + steps - 1, in dispatch order), the figures the line's
    roofline divides by."""
    import sqlite3
    c = sqlite3.connect(db)
    rows = c.execute("select s.display_name, d.start, d.end from rocpd_kernel_dispatch d join kernel_symbols s "
                     "on d.kernel_id = s.id order by d.start").fetchall()
    per = {}
    for name, t0, t1 in rows:
        per.setdefault(name, []).append((t1 - t0) / 1e3)
    srcs = ["block_scaled_fp8_x128_amd/csrc/" + f for f in sorted(os.listdir(os.path.join(ROOT, "block_scaled_fp8_x128_amd",
                                                                                      "csrc")))]
    title = "`bench.py` default run" if workload == "all" else "`bench.py --workload %s`" % workload
    lines = ["# rocprofv3 kernel trace: " + title, "",
             "Command (on an MI355X, from the repository root):", "", "    " + command, "",
             "Sources at the time of the trace (sha256, first 16 hex digits):", ""]
    lines += ["- `%s`: %s" % (f, src_hash(os.path.join(ROOT, f))) for f in srcs]
    lines += ["- `bench.py`: %s" % src_hash(os.path.join(ROOT, "bench.py")), ""]
    dom = DOMINANT["dense"][0]
    heads = [d for (n, t0, t1), d in zip(rows, [(r[2] - r[1]) / 1e3 for r in rows])
             if n.startswith("void " + dom) or n.startswith(dom)]
    first = heads[4 * warmup: 4 * (warmup + steps)] if workload in ("all", "dense") else []
    if first:
        srt = sorted(first)
        lines += ["## Headline kernel, timed dispatches", "",
                  "`%s`: the dense layer's QKV, gate+up, down and o_proj GEMMs of the %d timed steps (the first %d "
                  "dispatches of the kernel are the warm-up steps)." % (dom, steps, 4 * warmup), "",
                  "| dispatches | mean us | median us | min us | max us |", "|---|---|---|---|---|",
                  "| %d | %.1f | %.1f | %.1f | %.1f |" % (len(first), sum(first) / len(first), srt[len(srt) // 2],
                                                         srt[0], srt[-1]), ""]
    lines += ["## All kernels", "", "| kernel | calls | total ms | mean us | median us | min us |",
              "|---|---|---|---|---|---|"]
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        v2 = sorted(v)
        short = name.replace("void ", "").split("(")[0].replace("|", "/")
        lines.append("| `%s` | %d | %.3f | %.1f | %.1f | %.1f |" % (short, len(v), sum(v) / 1e3, sum(v) / len(v),
                                                                  v2[len(v2) // 2], v2[0]))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines[:40]))


def summarize_counters(db, command, out):
    """Markdown table of a rocprofv3 --pmc database of SQ / GRBM counters: per kernel the
    dispatches, mean duration and the derived rates (where their counters were collected):
    - clock = GRBM_GUI_ACTIVE / 8 XCDs / dispatch duration;
    - MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8);
    - VALU active = SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES;
    - LDS indexed = SQ_LDS_IDX_ACTIVE / SQ_BUSY_CU_CYCLES;
    - wait = SQ_WAIT_ANY / SQ_WAVE_CYCLES (waves stalled on a memory count or the barrier)."""
    import sqlite3
    c = sqlite3.connect(db)
    per = {}
    for kname, cname, val, did, t0, t1 in c.execute("select kernel_name, counter_name, value, dispatch_id, start, end "
                                                    "from counters_collection"):
        d = per.setdefault(kname, {}).setdefault(did, {"dur_us": (t1 - t0) / 1e3})
        d[cname] = d.get(cname, 0.0) + val
    names = sorted({n for k in per.values() for d in k.values() for n in d if n != "dur_us"})

    def mean(k, name):
        v = [d[name] for d in per[k].values() if name in d]
        return sum(v) / len(v) if v else None

    def ratio(a, b, scale=1.0):
        return None if a is None or not b else a / (b * scale)

    lines = ["# rocprofv3 counters per kernel", "", "Command (on an MI355X, from the repository root):", "",
             "    " + command, "", "Counters: " + ", ".join("`%s`" % n for n in names), "",
             "Sources at the time of the run (sha256, first 16 hex digits):", ""]
    srcs = ["block_scaled_fp8_x128_amd/csrc/" + f for f in sorted(os.listdir(os.path.join(ROOT, "block_scaled_fp8_x128_amd",
                                                                                      "csrc")))]
    lines += ["- `%s`: %s" % (f, src_hash(os.path.join(ROOT, f))) for f in srcs + ["bench.py"]]
    lines += ["", "| kernel | dispatches | mean us | clock MHz | MFMA busy | VALU active | LDS indexed | "
                  "LDS bank conflicts | wait |", "|---|---|---|---|---|---|---|---|---|"]
    order = sorted(per, key=lambda k: -sum(d["dur_us"] for d in per[k].values()))
    fmt = lambda v, pct=True: "-" if v is None else ("%.1f%%" % (100 * v) if pct else "%.0f" % v)  # noqa: E731
    for k in order[:12]:
        dur = mean(k, "dur_us")
        gui = mean(k, "GRBM_GUI_ACTIVE")
        clock = None if gui is None or dur < 20 else gui / 8 / dur
        mfma = ratio(mean(k, "SQ_VALU_MFMA_BUSY_CYCLES"), gui, 1024 / 8)
        valu = ratio(mean(k, "SQ_ACTIVE_INST_VALU"), mean(k, "SQ_WAVE_CYCLES"))
        lds = ratio(mean(k, "SQ_LDS_IDX_ACTIVE"), mean(k, "SQ_BUSY_CU_CYCLES"))
        wait = ratio(mean(k, "SQ_WAIT_ANY"), mean(k, "SQ_WAVE_CYCLES"))
        short = k.replace("void ", "").split("(")[0].replace("|", "/")
        lines.append("| `%s` | %d | %.1f | %s | %s | %s | %s | %s | %s |" % (
            short, len(per[k]), dur, fmt(clock, False), fmt(mfma), fmt(valu), fmt(lds),
            fmt(mean(k, "SQ_LDS_BANK_CONFLICT"), False), fmt(wait)))
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# ---------------------------------------------------------------------------
# main
# ---------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="all", choices=["all", "dense", "recal", "decode", "moe", "train"])
    ap.add_argument("--mode", type=int, default=0, help="scale mode: 0 EXACT, 1 POW2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DB", "WRITE_DB"))
    ap.add_argument("--pmc-command", default="", help="the profiled command, recorded with --summarize-pmc")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DB", "OUT_MD"),
                    help="summarize a rocprofv3 --kernel-trace database of this script (with --workload)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("PMC_DB", "OUT_MD"),
                    help="summarize a rocprofv3 --pmc database of SQ / GRBM counters")
    args = ap.parse_args()
    if args.summarize_counters:
        summarize_counters(args.summarize_counters[0], args.pmc_command, args.summarize_counters[1])
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload, args.pmc_command)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace[0], args.pmc_command, args.steps, args.warmup, args.summarize_trace[1],
                        args.workload)
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

    if args.workload == "all":
        # the headline: the 8B-shaped dense layer (EXACT); then every other row, each timed on its own
        cpu_on = not args.no_cpu_baseline
        bufs = dense_data(dev)
        flops = sum(2.0 * b["M"] * b["N"] * b["K"] for b in bufs)
        ms = timed_loop(dense_step(fp8bs, bufs, 0), args.steps, args.warmup, timer)
        kernels, roof = summarize_dense(bufs, timer)
        out = {"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOP/s", **common,
               "ms_per_step": round(ms, 4), "dtype": "fp8e4m3",
               "config": {"workload": "8B-shaped dense layer at M=8192 tokens: recalibrate 4 weights (128x128, one "
                                      "batched launch), quantize 4 inputs (1x128), GEMMs QKV K4096 N6144, gate+up "
                                      "K4096 N28672, down K14336 N4096, o_proj K4096 N4096",
                          "scale_mode": "exact", "out_dtype": "bf16", "gemm_flops_per_step": flops},
               "roofline": roof, "kernels": with_spread(kernels, timer)}
        log("d3 dense, POW2")
        rows = {"d3_dense_pow2": row_dense_pow2(fp8bs, bufs, args.steps, args.warmup)}
        del bufs
        torch.cuda.empty_cache()
        if cpu_on:
            log("timing the oracle: dense")
            out["cpu_baseline"] = cpu_dense()
        for key, fn in (("d1_recal", row_recal), ("d2_quant_act", row_quant_act), ("d4_decode", row_decode),
                        ("d5_moe", row_moe), ("d6_tiny", row_tiny), ("next2_gemm_quant", row_gemm_quant),
                        ("next4_kv_attention", row_attention)):
            log("row " + key)
            rows[key] = fn(fp8bs, dev, args.steps, args.warmup, cpu_on)
            torch.cuda.empty_cache()
        out["rows"] = rows
        print(json.dumps(out), flush=True)
        return
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
        kernels, roof = summarize_train(bufs, timer, args.mode)
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
        step.stream(None, 1)
        step.stream(timer, args.steps)
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
            kernels["gemm_stream_" + p["name"]] = hbm_entry(timer.avg_ms("gemm5_" + p["name"]) / 5, gbytes)
        # the step's longest GEMM: gate+up at the largest M (the persistent 128x256 kernel), timed as
        # five back-to-back launches on rotated weight copies
        big = max(pairs, key=lambda p: p["N"] * p["K"] + p["M"])
        tb = timer.avg_ms("gemm5_" + big["name"]) / 5
        nb = big["N"] * big["K"] * (1 + 4 / 16384) + big["M"] * big["K"] * (1 + 4 / 128) + big["M"] * big["N"] * 2
        ach = nb / (tb * 1e-3) / 1e9
        out = {"metric": METRIC, "value": round(flops / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s", **common,
               "ms_per_step": round(ms, 4), "dtype": "fp8e4m3",
               "config": {"workload": "rollout decode: M in {1,16,64,256} x (gate+up K4096 N28672, down K14336 "
                                      "N4096), fp8_block_linear from bf16 activations (quantized inside the GEMM "
                                      "for M <= 16), 5 rotated weight copies"},
               "roofline": {"kernel": "fp8_block_gemm (persistent 128x256 kernel), %s" % big["name"],
                            "bound": "hbm",
                            "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": None},
               "kernels": kernels}
        cpu = None
    else:
        step, shapes, flops, E = moe_workload(fp8bs, dev, args.mode)
        ms = timed_loop(step, args.steps, args.warmup, timer)
        step.gather_form(None, 2)
        step.gather_form(timer, args.steps)
        torch.cuda.synchronize()
        kernels = {}
        for name, (m, n, k) in shapes.items():
            t = timer.avg_ms("grouped_" + name)
            nbytes = m * k + m * k // 128 * 4 + E * n * k * (1 + 4 / 16384) + m * n * 2
            kernels["grouped_" + name] = {**mfma_entry(t, 2.0 * m * n * k), **hbm_entry(t, nbytes)}
        m, _, k = shapes["gate_up"]
        # dispatch quantizer: the token rows read once (T x K bf16), the routing, codes and scales written
        for dname in ("quant_act_scatter_gate_up", "quant_act_gather_gate_up"):
            kernels[dname] = hbm_entry(timer.avg_ms(dname), T_TOKENS * k * 2 + m * 4 + m * k + m * k // 128 * 4)
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
                                      "(65536 rows); the dispatch quantizing each token row once into its 8 expert rows, grouped "
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
