"""Benchmark of the block-FP8 linear-layer hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input.
Workloads (--workload):
  dense  (default) 8B-shaped dense layer at M = 8192 tokens: per-step
         recalibration of the layer's four weights (128x128 quantizer), the
         1x128 quantization of each GEMM input, and the four block-scaled
         GEMMs QKV (K 4096, N 6144), gate+up (K 4096, N 28672),
         down (K 14336, N 4096), o_proj (K 4096, N 4096).
  recal  per-step recalibration of 32 layers x 4 weights, EXACT then POW2.
  decode rollout decode: M in {1, 16, 64, 256} against the gate+up and down
         weights, activations quantized on the fly.
  moe    MoE layer: 128 experts, hidden 2048, expert FFN 768, 8192 tokens
         routed top-8: expert-weight recalibration, quantization of the
         gate+up and down inputs, the two grouped GEMMs.
Prints ONE JSON line.  `value` is GEMM TFLOP/s over the whole step
(quantizers included) except for `recal` (GB/s); per-kernel times come from
HIP events on the stream the kernels run on.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

METRIC = "block-FP8 GEMM TFLOP/s (% of FP8 MFMA peak); quantizer GB/s (% of HBM peak)"
PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (published)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published)

DENSE = [("qkv", 6144, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336), ("o_proj", 4096, 4096)]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def bf16_dev(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


class KernelTimer:
    """Per-kernel HIP-event timing on torch's current stream (the library's stream)."""

    def __init__(self):
        self.pairs = {}

    def run(self, name, fn):
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

    def reset(self):
        self.pairs = {}


def timed_loop(step, steps, warmup, timer):
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


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

def dense_workload(fp8bs, dev, mode):
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

    def step(timer):
        for b in bufs:
            maybe(timer, "quant_w_" + b["name"], lambda: fp8bs.quant_w_128x128(b["w"], mode, out=(b["wq"], b["ws"])))
        for b in bufs:
            maybe(timer, "quant_act_" + b["name"], lambda: fp8bs.quant_act_1x128(b["x"], mode, out=(b["xq"], b["xs"])))
            maybe(timer, "gemm_" + b["name"],
                  lambda: fp8bs.fp8_block_gemm(b["xq"], b["xs"], b["wq"], b["ws"], out=b["y"]))

    flops = sum(2.0 * b["M"] * b["N"] * b["K"] for b in bufs)
    return step, bufs, flops


def summarize_dense(bufs, timer, ms_step, flops):
    kernels = {}
    for b in bufs:
        M, N, K = b["M"], b["N"], b["K"]
        t = timer.avg_ms("gemm_" + b["name"])
        tf = 2.0 * M * N * K / (t * 1e-3) / 1e12
        kernels["gemm_" + b["name"]] = {"ms": round(t, 4), "TFLOP/s": round(tf, 1),
                                        "frac_fp8_peak": round(tf / PEAK_FP8_TFLOPS, 4)}
        for q, R, C in (("quant_act_", M, K), ("quant_w_", N, K)):
            tq = timer.avg_ms(q + b["name"])
            nbytes = R * C * 3 + (R * C // (128 if q == "quant_act_" else 16384)) * 4
            gbs = nbytes / (tq * 1e-3) / 1e9
            kernels[q + b["name"]] = {"ms": round(tq, 4), "GB/s": round(gbs, 1),
                                      "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}
    g = bufs[1]  # gate+up: the largest GEMM, most of the step's FLOPs
    t = timer.avg_ms("gemm_gate_up")
    ach = 2.0 * g["M"] * g["N"] * g["K"] / (t * 1e-3) / 1e12
    roof = {"kernel": "gemm_kernel (gate+up, M8192 N28672 K4096)", "bound": "mfma", "achieved": round(ach, 1),
            "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(ach / PEAK_FP8_TFLOPS, 4), "traffic": None}
    return kernels, roof


def cpu_baseline_dense(target_s=12.0):
    """The oracle GEMM (exact per-block sums, fp64 scales) on a bounded sample
    of the gate+up GEMM: the first R rows of Y, R sized for ~target_s."""
    import oracle
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
            "sample": "gate+up GEMM, first %d of 8192 rows (N 28672, K 4096), %.1f s" % (rows, dt)}


def recal_workload(fp8bs, dev):
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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="dense", choices=["dense", "recal"])
    ap.add_argument("--mode", type=int, default=0, help="scale mode: 0 EXACT, 1 POW2")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(every kernel runs on one GPU's share at its real shape); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import block_scaled_fp8_x128_amd as fp8bs
    if not os.path.exists(fp8bs.LIB_PATH):
        from block_scaled_fp8_x128_amd import build
        build.build()
    fp8bs.lib()
    dev = torch.device("cuda", 0)
    timer = KernelTimer()

    if args.workload == "dense":
        step, bufs, flops = dense_workload(fp8bs, dev, args.mode)
        ms = timed_loop(step, args.steps, args.warmup, timer)
        kernels, roof = summarize_dense(bufs, timer, ms, flops)
        value = flops / (ms * 1e-3) / 1e12
        out = {"metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "fp8e4m3", "data": "synthetic",
               "config": {"workload": "8B-shaped dense layer at M=8192 tokens: recalibrate 4 weights (128x128), "
                                      "quantize 4 inputs (1x128), GEMMs QKV K4096 N6144, gate+up K4096 N28672, "
                                      "down K14336 N4096, o_proj K4096 N4096",
                          "scale_mode": "pow2" if args.mode else "exact", "out_dtype": "bf16",
                          "gemm_flops_per_step": flops},
               "roofline": roof, "kernels": kernels}
        if not args.no_cpu_baseline:
            log("timing the oracle on the host (bounded sample)")
            out["cpu_baseline"] = cpu_baseline_dense()
    else:
        step, nbytes = recal_workload(fp8bs, dev)
        ms = timed_loop(step, args.steps, args.warmup, timer)
        te, tp = timer.avg_ms("recal_exact"), timer.avg_ms("recal_pow2")
        gbs = 2 * nbytes / (ms * 1e-3) / 1e9
        out = {"metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
               "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
               "vs_baseline": None, "dtype": "bf16->fp8e4m3", "data": "synthetic",
               "config": {"workload": "per-step recalibration: 32 layers x {6144x4096, 4096x4096, 28672x4096, "
                                      "4096x14336} bf16 weights, 128x128 blocks, EXACT then POW2",
                          "bytes_per_pass": nbytes},
               "roofline": {"kernel": "quant_w_kernel (batched)", "bound": "hbm",
                            "achieved": round(nbytes / (te * 1e-3) / 1e9, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(nbytes / (te * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "traffic": None},
               "kernels": {"recal_exact": {"ms": round(te, 4)}, "recal_pow2": {"ms": round(tp, 4)}}}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
