"""CPU oracle of the block-wise FP8 linear layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product library
(``block_scaled_fp8_x128_amd``) never imports it, and it never imports the
product library: the two share no code.  Inputs come from ``synth``.

This module is argument marshalling (numpy <-> ctypes) around the plain C
definitions in ``fp8bs_oracle.c``; every arithmetic step lives there, with
the passage of the article each one follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp8bs_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

SCALE_EXACT = 0
SCALE_POW2 = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, no FMA contraction, no fast-math)."""
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-std=c99",
               "-Wall", "-Wextra", "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, LIB)
    return LIB


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            build()
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint32]
        L.oracle_e4m3_encode.restype = ctypes.c_uint32
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode_array.argtypes = [P, I64, P]
        L.oracle_e4m3_decode_array.argtypes = [P, I64, P]
        L.oracle_block_scale.restype = ctypes.c_float
        L.oracle_block_scale.argtypes = [ctypes.c_float, ctypes.c_int]
        L.oracle_quant_act_1x128.argtypes = [P, I64, I64, P, P, ctypes.c_int]
        L.oracle_quant_w_128x128.argtypes = [P, I64, I64, P, P, ctypes.c_int]
        L.oracle_bf16_from_double.restype = ctypes.c_uint16
        L.oracle_bf16_from_double.argtypes = [ctypes.c_double]
        L.oracle_swiglu_bf16.argtypes = [P, I64, I64, P]
        L.oracle_swiglu_quant_1x128.argtypes = [P, I64, I64, P, P, ctypes.c_int]
        L.oracle_gemm.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.oracle_gemm_sampled.argtypes = [P, P, P, P, I64, I64, I64, P, P, I64, P]
        L.oracle_gemm_1x128.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.oracle_gemm_1x128_sampled.argtypes = [P, P, P, P, I64, I64, I64, P, P, I64, P]
        L.oracle_grouped_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P]
        L.oracle_grouped_gemm_sampled.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, P, I64, P]
        L.oracle_e4m3_x512_table.argtypes = [P]
        for f in (L.oracle_gemm_full, L.oracle_gemm_1x128_full):
            f.restype = ctypes.c_int
            f.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.oracle_grouped_gemm_full.restype = ctypes.c_int
        L.oracle_grouped_gemm_full.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P]
        L.oracle_kv_attention_decode.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_double, P]
        L.oracle_max_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError("expected %s, got %s" % (np.dtype(dtype), a.dtype))
    return a


def max_threads() -> int:
    return int(lib().oracle_max_threads())


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


# ---- E4M3 codec ----------------------------------------------------------------

def e4m3_decode(code: int) -> float:
    return float(lib().oracle_e4m3_decode(int(code)))


def e4m3_encode(v: float) -> int:
    return int(lib().oracle_e4m3_encode(float(v)))


def e4m3_encode_array(v) -> np.ndarray:
    v = _c(v, np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(v), v.size, _ptr(out))
    return out


def e4m3_decode_array(c) -> np.ndarray:
    c = _c(c, np.uint8)
    out = np.empty(c.shape, dtype=np.float64)
    lib().oracle_e4m3_decode_array(_ptr(c), c.size, _ptr(out))
    return out


def block_scale(amax: float, mode: int = SCALE_EXACT) -> float:
    """fp32 dequantization scale of a block with largest magnitude ``amax``."""
    return float(lib().oracle_block_scale(float(amax), int(mode)))


# ---- quantizers ----------------------------------------------------------------

def quant_act_1x128(x_bf16, mode: int = SCALE_EXACT):
    """x_bf16: uint16 [M, K] -> (codes uint8 [M, K], scales fp32 [M, K/128])."""
    x = _c(x_bf16, np.uint16)
    M, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 128), dtype=np.float32)
    lib().oracle_quant_act_1x128(_ptr(x), M, K, _ptr(q), _ptr(s), int(mode))
    return q, s


def bf16_from_double(v: float) -> int:
    """Nearest bf16 payload (ties to even) of a double."""
    return int(lib().oracle_bf16_from_double(float(v)))


def swiglu_bf16(gu_bf16) -> np.ndarray:
    """gu_bf16: uint16 [M, 2F] (gate columns, then up columns) -> h bf16 payloads [M, F],
    h = RN_bf16((g * sigma(g)) * u) evaluated in fp64."""
    gu = _c(gu_bf16, np.uint16)
    M, F2 = gu.shape
    if F2 % 2:
        raise ValueError("gu must have an even number of columns")
    h = np.empty((M, F2 // 2), dtype=np.uint16)
    lib().oracle_swiglu_bf16(_ptr(gu), M, F2 // 2, _ptr(h))
    return h


def swiglu_quant_1x128(gu_bf16, mode: int = SCALE_EXACT):
    """The gated activation of gu [M, 2F], then quant_act_1x128: (codes [M, F], scales [M, F/128])."""
    gu = _c(gu_bf16, np.uint16)
    M, F2 = gu.shape
    F = F2 // 2
    if F2 % 2 or F % 128:
        raise ValueError("gu must be [M, 2F] with F a multiple of 128")
    q = np.empty((M, F), dtype=np.uint8)
    s = np.empty((M, F // 128), dtype=np.float32)
    lib().oracle_swiglu_quant_1x128(_ptr(gu), M, F, _ptr(q), _ptr(s), int(mode))
    return q, s


def quant_w_128x128(w_bf16, mode: int = SCALE_EXACT):
    """w_bf16: uint16 [N, K] -> (codes uint8 [N, K], scales fp32 [N/128, K/128])."""
    w = _c(w_bf16, np.uint16)
    N, K = w.shape
    if N % 128 or K % 128:
        raise ValueError("N and K must be multiples of 128")
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((N // 128, K // 128), dtype=np.float32)
    lib().oracle_quant_w_128x128(_ptr(w), N, K, _ptr(q), _ptr(s), int(mode))
    return q, s


def quant_act_1x128_gather(x_bf16, rows, mode: int = SCALE_EXACT):
    """quant_act_1x128 of the gathered rows x[rows] (MoE dispatch: token rows in
    expert order, a token repeated once per expert it is routed to).
    x_bf16: uint16 [T, K]; rows: int [M] in [0, T) -> (codes [M, K], scales [M, K/128]).
    The gather is numpy's; every arithmetic step is the quantizer's."""
    x = _c(x_bf16, np.uint16)
    r = np.asarray(rows, dtype=np.int64)
    if r.size and (r.min() < 0 or r.max() >= x.shape[0]):
        raise ValueError("row index out of range")
    return quant_act_1x128(x[r].reshape(r.size, x.shape[1]), mode)


def quant_act_1x128_t(x_bf16, mode: int = SCALE_EXACT):
    """quant_act_1x128 of X^T: 1x128 blocks down the columns of X [M, K], written as
    codes [K, M] and scales [K, M/128] (the weight gradient's operands)."""
    return quant_act_1x128(np.ascontiguousarray(np.asarray(x_bf16).T), mode)


# ---- GEMMs ---------------------------------------------------------------------

def gemm(xq, xs, wq, ws) -> np.ndarray:
    """fp64 Y [M, N] = block-scaled Xq Wq^T."""
    xq = _c(xq, np.uint8)
    wq = _c(wq, np.uint8)
    xs = _c(xs, np.float32)
    ws = _c(ws, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y))
    return y


def gemm_sampled(xq, xs, wq, ws, rows, cols) -> np.ndarray:
    xq = _c(xq, np.uint8)
    wq = _c(wq, np.uint8)
    xs = _c(xs, np.float32)
    ws = _c(ws, np.float32)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty(rows.shape, dtype=np.float64)
    lib().oracle_gemm_sampled(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K,
                              _ptr(rows), _ptr(cols), rows.size, _ptr(y))
    return y


def gemm_1x128(xq, xs, wq, ws) -> np.ndarray:
    """fp64 Y [M, N] with 1x128 scales on both operands: ws [N, K/128]."""
    xq, wq = _c(xq, np.uint8), _c(wq, np.uint8)
    xs, ws = _c(xs, np.float32), _c(ws, np.float32)
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    lib().oracle_gemm_1x128(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y))
    return y


def gemm_1x128_sampled(xq, xs, wq, ws, rows, cols) -> np.ndarray:
    xq, wq = _c(xq, np.uint8), _c(wq, np.uint8)
    xs, ws = _c(xs, np.float32), _c(ws, np.float32)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty(rows.shape, dtype=np.float64)
    lib().oracle_gemm_1x128_sampled(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K,
                                    _ptr(rows), _ptr(cols), rows.size, _ptr(y))
    return y


def grouped_gemm(xq, xs, wq, ws, offsets) -> np.ndarray:
    """fp64 Y [M_total, N]; wq [E, N, K], ws [E, N/128, K/128], offsets int32 [E+1]."""
    xq = _c(xq, np.uint8)
    wq = _c(wq, np.uint8)
    xs = _c(xs, np.float32)
    ws = _c(ws, np.float32)
    offs = _c(np.asarray(offsets, dtype=np.int32), np.int32)
    M, K = xq.shape
    E, N, _ = wq.shape
    y = np.empty((M, N), dtype=np.float64)
    lib().oracle_grouped_gemm(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(offs), E, M, N, K, _ptr(y))
    return y


def grouped_gemm_sampled(xq, xs, wq, ws, offsets, rows, cols) -> np.ndarray:
    xq = _c(xq, np.uint8)
    wq = _c(wq, np.uint8)
    xs = _c(xs, np.float32)
    ws = _c(ws, np.float32)
    offs = _c(np.asarray(offsets, dtype=np.int32), np.int32)
    rows = _c(np.asarray(rows, dtype=np.int64), np.int64)
    cols = _c(np.asarray(cols, dtype=np.int64), np.int64)
    M, K = xq.shape
    E, N, _ = wq.shape
    y = np.empty(rows.shape, dtype=np.float64)
    lib().oracle_grouped_gemm_sampled(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(offs), E, M, N, K,
                                      _ptr(rows), _ptr(cols), rows.size, _ptr(y))
    return y


# ---- the same GEMMs, every output, at full configuration sizes -----------------
# Codes decoded once through a table of decode(c) * 2^9; each 128-wide block's
# dot product summed in fp64, which is exact (all partial sums are integers
# below 2^43), so the outputs are bit-identical to gemm / gemm_1x128 /
# grouped_gemm above.

def e4m3_x512_table() -> np.ndarray:
    """The full-output GEMMs' table: decode(c) * 2^9 for c = 0 .. 255 (NaN codes NaN)."""
    t = np.empty(256, dtype=np.float64)
    lib().oracle_e4m3_x512_table(_ptr(t))
    return t


def _full(fn, xq, xs, wq, ws, ncols_of_w):
    xq, wq = _c(xq, np.uint8), _c(wq, np.uint8)
    xs, ws = _c(xs, np.float32), _c(ws, np.float32)
    M, K = xq.shape
    N = ncols_of_w(wq)
    y = np.empty((M, N), dtype=np.float64)
    if fn(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y)) != 0:
        raise MemoryError("oracle: no memory for the decoded operands")
    return y


def gemm_full(xq, xs, wq, ws) -> np.ndarray:
    """gemm(), every output, bit-identical, fast enough for the 8B-shaped layers."""
    return _full(lib().oracle_gemm_full, xq, xs, wq, ws, lambda w: w.shape[0])


def gemm_1x128_full(xq, xs, wq, ws) -> np.ndarray:
    """gemm_1x128(), every output, bit-identical."""
    return _full(lib().oracle_gemm_1x128_full, xq, xs, wq, ws, lambda w: w.shape[0])


def grouped_gemm_full(xq, xs, wq, ws, offsets) -> np.ndarray:
    """grouped_gemm(), every output, bit-identical."""
    xq, wq = _c(xq, np.uint8), _c(wq, np.uint8)
    xs, ws = _c(xs, np.float32), _c(ws, np.float32)
    offs = _c(np.asarray(offsets, dtype=np.int32), np.int32)
    M, K = xq.shape
    E, N, _ = wq.shape
    y = np.empty((M, N), dtype=np.float64)
    if lib().oracle_grouped_gemm_full(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(offs), E, M, N, K,
                                      _ptr(y)) != 0:
        raise MemoryError("oracle: no memory for the decoded operands")
    return y


# ---- attention over an FP8 KV cache ---------------------------------------------

def kv_attention_decode(q_bf16, kq, ks, vq, vs, lens, sm_scale: float) -> np.ndarray:
    """fp64 o [B, Hq, 128]: one query token per sequence attending to its first lens[b]
    cached tokens; q bf16 payloads [B, Hq, 128], kq / vq codes [B, T, Hkv, 128], ks / vs
    fp32 [B, T, Hkv], lens int32 [B]."""
    q = _c(q_bf16, np.uint16)
    kq, vq = _c(kq, np.uint8), _c(vq, np.uint8)
    ks, vs = _c(ks, np.float32), _c(vs, np.float32)
    lens = _c(np.asarray(lens, dtype=np.int32), np.int32)
    B, Hq, D = q.shape
    _, T, Hkv, D2 = kq.shape
    if D != 128 or D2 != 128 or Hq % Hkv or vq.shape != kq.shape or ks.shape != (B, T, Hkv) or \
            vs.shape != ks.shape or lens.shape != (B,):
        raise ValueError("shapes do not match")
    out = np.empty((B, Hq, D), dtype=np.float64)
    lib().oracle_kv_attention_decode(_ptr(q), _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs), _ptr(lens), B, T, Hq, Hkv,
                                     float(sm_scale), _ptr(out))
    return out
