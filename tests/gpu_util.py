"""Helpers of the GPU parity tests: device transfers and the GEMM gate.

The GEMM gate: max |Y_gpu - Y_oracle| <= 1e-2 * rms(Y_oracle), applied to the
library's fp32 output mode, with the oracle's fp64 result from the oracle's
own quantization of the same seeded bf16 inputs.
"""

import sys

import numpy as np
import torch

GEMM_TOL = 1e-2
# Internal precision of the FP8 matrix-core dot product: the 128 products of
# a K block are not summed exactly; measured deviations stay below 2^-12 of
# the block's sum of |products| (a pin in test_gpu_train checks 2^-11 on
# crafted worst cases).  Used where both operands carry outliers.
MFMA_DOT_TAU = 2.0 ** -11


def dev():
    return torch.device("cuda", 0)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_to_dev(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_bitexact(name, got: np.ndarray, ref: np.ndarray):
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    g = got.view(np.uint8) if got.dtype == np.uint8 else got.view(np.uint32)
    r = ref.view(np.uint8) if ref.dtype == np.uint8 else ref.view(np.uint32)
    bad = np.nonzero((g != r).reshape(-1))[0]
    assert bad.size == 0, "%s: %d mismatches, first at flat index %d: got %r want %r" % (
        name, bad.size, bad[0], got.reshape(-1)[bad[0]], ref.reshape(-1)[bad[0]])


def gemm_gate(name, y_gpu: np.ndarray, y_ref: np.ndarray, tol: float = GEMM_TOL):
    """max |err| <= tol * rms(oracle); returns (max_err / rms)."""
    rms = float(np.sqrt(np.mean(np.square(y_ref))))
    err = float(np.max(np.abs(y_gpu.astype(np.float64) - y_ref))) if y_ref.size else 0.0
    rel = err / rms if rms > 0 else err
    say("%s: max|err| = %.3e, rms = %.3e, max|err|/rms = %.3e" % (name, err, rms, rel))
    assert np.isfinite(y_gpu).all()
    assert err <= tol * rms, (name, err, rms)
    return rel


def sample_positions(M, N, count, seed=0, block=128):
    """Output positions for sampled checks: every corner, the full mesh of tile-edge
    rows x tile-edge columns (the first and last row and column of every 128-wide
    tile), one random position inside every 128x128 tile, then `count` random ones."""
    g = np.random.default_rng(seed)
    edge_r = sorted({0, M - 1} | {min(M - 1, r) for k in range(1, M // block + 1) for r in (k * block - 1, k * block)})
    edge_c = sorted({0, N - 1} | {min(N - 1, c) for k in range(1, N // block + 1) for c in (k * block - 1, k * block)})
    rr, cc = np.meshgrid(np.array(edge_r, np.int64), np.array(edge_c, np.int64), indexing="ij")
    tr, tc = np.meshgrid(np.arange(0, M, block, dtype=np.int64), np.arange(0, N, block, dtype=np.int64),
                         indexing="ij")
    tr = np.minimum(tr + g.integers(0, block, tr.shape), M - 1)
    tc = np.minimum(tc + g.integers(0, block, tc.shape), N - 1)
    rows = [rr.reshape(-1), tr.reshape(-1), g.integers(0, M, count)]
    cols = [cc.reshape(-1), tc.reshape(-1), g.integers(0, N, count)]
    return np.concatenate(rows), np.concatenate(cols)


def gemm_gate_abs(name, y_gpu: np.ndarray, y_ref: np.ndarray, abs_sum: np.ndarray, tol: float = GEMM_TOL,
                  tau: float = MFMA_DOT_TAU):
    """Per element |err| <= tol * rms(oracle) + tau * abs_sum, abs_sum being the
    oracle's sum over K blocks of |scale product| * sum |decoded products| (the
    standard dot-product error bound, with the matrix core's internal
    precision as the relative factor).  Reports the plain max|err|/rms too."""
    rms = float(np.sqrt(np.mean(np.square(y_ref))))
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = tol * rms + tau * abs_sum
    say("%s: max|err|/rms = %.3e, max err/bound = %.3f" % (name, float(err.max()) / rms, float((err / bound).max())))
    assert np.isfinite(y_gpu).all()
    assert (err <= bound).all(), (name, int((err > bound).sum()))
