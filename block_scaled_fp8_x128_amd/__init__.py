"""Block-scaled FP8 linear layers for AMD MI355X (gfx950).

Thin Python binding of ``libfp8bs.so`` (C ABI in ``include/fp8bs.h``): each
function checks dtypes, shapes and devices, allocates outputs with torch (torch
is used for device memory and streams only) and passes raw pointers plus the
current HIP stream.  Every arithmetic step runs in the library's kernels; there
is no fallback: if the library is not built, loading it raises.

Method: the article "NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
precision training" (Jessie A Ellis, Apr 20 2026), section "Technical
breakthrough" -- block-wise E4M3 with 1x128 activation blocks and 128x128
weight blocks, FP8 math in linear layers; section "Real-world performance
gains" -- scales recalibrated after every step, MoE models; closing section --
power-of-2 scaling factors.
"""

from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfp8bs.so")

SCALE_EXACT = 0
SCALE_POW2 = 1
OUT_BF16 = 0
OUT_FP32 = 1
STATUS_SCRATCH_TOO_SMALL = 6
NOALLOC_SCRATCH_BYTES = 1 << 20  # FP8BS_NOALLOC_SCRATCH_BYTES

# The functions declared in include/fp8bs.h, in declaration order.
EXPORTS = (
    "quant_act_1x128",
    "quant_act_1x128_t",
    "quant_act_1x128_dual",
    "quant_act_1x128_gather",
    "quant_act_1x128_scatter",
    "swiglu_quant_1x128",
    "quant_w_128x128",
    "quant_w_128x128_batched",
    "quant_w_128x128_dual",
    "quant_w_128x128_dual_batched",
    "fp8_block_gemm",
    "fp8_block_gemm_1x128",
    "fp8_block_gemm_1x128_pow2",
    "fp8_block_grouped_gemm",
    "fp8_block_gemm_pow2",
    "fp8_block_grouped_gemm_pow2",
    "fp8_block_gemm_quant",
    "fp8bs_gemm_quant_workspace_size",
    "fp8_kv_attention_decode",
    "fp8bs_kv_attention_workspace_size",
    "fp8_block_grouped_gemm_noalloc",
    "fp8_block_linear",
    "fp8_block_linear_pow2",
    "fp8bs_linear_workspace_size",
    "fp8bs_gemm_workspace_size",
    "fp8bs_grouped_workspace_size",
    "fp8bs_status_string",
    "fp8bs_abi_version",
)

_lib = None


class Fp8bsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed with status %d: %s" % (fn, status, status_string(status)))


def lib() -> ctypes.CDLL:
    """Load libfp8bs.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libfp8bs.so is not built (run `python -m block_scaled_fp8_x128_amd.build`)")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
        L.quant_act_1x128.argtypes = [P, I64, I64, P, P, I32, P]
        L.quant_act_1x128_t.argtypes = [P, I64, I64, P, P, I32, P]
        L.quant_act_1x128_dual.argtypes = [P, I64, I64, P, P, P, P, I32, P]
        L.swiglu_quant_1x128.argtypes = [P, I64, I64, P, P, I32, P]
        L.quant_act_1x128_gather.argtypes = [P, I64, I64, P, I64, P, P, I32, P]
        L.quant_act_1x128_scatter.argtypes = [P, I64, I64, P, I64, I64, P, P, I32, P]
        L.fp8_block_gemm_1x128.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P]
        L.fp8_block_gemm_1x128_pow2.argtypes = L.fp8_block_gemm_1x128.argtypes
        L.quant_w_128x128.argtypes = [P, I64, I64, P, P, I32, P]
        L.quant_w_128x128_batched.argtypes = [I64, P, P, P, P, P, I32, P]
        L.quant_w_128x128_dual.argtypes = [P, I64, I64, P, P, P, P, I32, P]
        L.quant_w_128x128_dual_batched.argtypes = [I64, P, P, P, P, P, P, P, I32, P]
        L.fp8_block_gemm.argtypes = [P, P, P, P, I64, I64, I64, P, I32, P, SZ, P]
        L.fp8_block_grouped_gemm.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, I32, P, SZ, P]
        L.fp8_block_gemm_pow2.argtypes = L.fp8_block_gemm.argtypes
        L.fp8_block_grouped_gemm_pow2.argtypes = L.fp8_block_grouped_gemm.argtypes
        L.fp8_block_grouped_gemm_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, I64, P, I32, P]
        L.fp8_block_gemm_quant.argtypes = [P, P, P, P, I64, I64, I64, P, P, P, I32, P, SZ, P]
        L.fp8bs_gemm_quant_workspace_size.argtypes = [I64, I64, I64]
        L.fp8bs_gemm_quant_workspace_size.restype = SZ
        L.fp8_kv_attention_decode.argtypes = [P, P, P, P, P, P, I64, I64, I64, I64, ctypes.c_float, P, I32, P, SZ, P]
        L.fp8bs_kv_attention_workspace_size.argtypes = [I64, I64, I64, I64]
        L.fp8bs_kv_attention_workspace_size.restype = SZ
        L.fp8_block_linear.argtypes = [P, P, P, I64, I64, I64, P, I32, P, SZ, P]
        L.fp8_block_linear_pow2.argtypes = L.fp8_block_linear.argtypes
        L.fp8bs_linear_workspace_size.argtypes = [I64, I64, I64]
        L.fp8bs_linear_workspace_size.restype = SZ
        L.fp8bs_gemm_workspace_size.argtypes = [I64, I64, I64]
        L.fp8bs_gemm_workspace_size.restype = SZ
        L.fp8bs_grouped_workspace_size.argtypes = [I64, I64, I64, I64]
        L.fp8bs_grouped_workspace_size.restype = SZ
        L.fp8bs_status_string.argtypes = [I32]
        L.fp8bs_status_string.restype = ctypes.c_char_p
        L.fp8bs_abi_version.restype = I32
        for fn in ("quant_act_1x128", "quant_act_1x128_t", "quant_act_1x128_dual", "swiglu_quant_1x128",
                   "quant_act_1x128_gather", "quant_act_1x128_scatter",
                   "fp8_block_gemm_1x128", "fp8_block_gemm_1x128_pow2", "quant_w_128x128", "quant_w_128x128_batched", "quant_w_128x128_dual",
                   "quant_w_128x128_dual_batched", "fp8_block_gemm",
                   "fp8_block_grouped_gemm", "fp8_block_gemm_pow2", "fp8_block_grouped_gemm_pow2",
                   "fp8_block_grouped_gemm_noalloc", "fp8_block_gemm_quant", "fp8_kv_attention_decode",
                   "fp8_block_linear", "fp8_block_linear_pow2"):
            getattr(L, fn).restype = I32
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fp8bs_status_string(int(status)).decode()


def abi_version() -> int:
    return int(lib().fp8bs_abi_version())


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise Fp8bsError(fn, status)


# The raw handle of the device's current stream.  torch's internal query skips
# building a Stream object: measured on the MI355X, 0.08 us against 1.9 us per
# call, which is most of a small launch's host time.  The public query is used
# where that entry is missing.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(t: torch.Tensor):
    if _raw_stream is not None:
        return _raw_stream(t.get_device())
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    # (a plain int: every pointer argument is declared c_void_p, which takes it as is)
    return t.data_ptr() if t is not None else None


def _bf16_payload(x: torch.Tensor, name: str) -> torch.Tensor:
    if x.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError("%s must be bfloat16 (or its 16-bit payload), got %s" % (name, x.dtype))
    if not x.is_cuda:
        raise ValueError("%s must be on a HIP device" % name)
    if not x.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return x


def _codes(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
        raise TypeError("%s must hold E4M3 codes (uint8 or float8_e4m3fn), got %s" % (name, t.dtype))
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous device tensor" % name)
    return t


def _f32(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype != torch.float32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError("%s must be a contiguous float32 device tensor" % name)
    return t


_CODE_DTYPES = (torch.uint8, torch.float8_e4m3fn)


def _out(t, shape, dtypes, device, name, what=None) -> torch.Tensor:
    """A caller-provided output: the C ABI receives no output sizes, so the
    kernels would write past an undersized or mistyped buffer; check it here.
    (The message is formatted only on failure: `name (what)`.)"""
    if not (isinstance(t, torch.Tensor) and t.dtype in dtypes and t.shape == tuple(shape) and t.device == device
            and t.is_contiguous()):
        label = name if what is None else "%s (%s)" % (name, what)
        if not isinstance(t, torch.Tensor):
            raise ValueError("%s must be a torch.Tensor" % label)
        if t.dtype not in dtypes:
            raise ValueError("%s must have dtype %s, got %s" % (label, " or ".join(map(str, dtypes)), t.dtype))
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s must have shape %s, got %s" % (label, tuple(shape), tuple(t.shape)))
        if t.device != device:
            raise ValueError("%s must be on %s, got %s" % (label, device, t.device))
        raise ValueError("%s must be contiguous" % label)
    return t


def _pair_out(out, M, K, device, nq="xq", ns="xs"):
    """(codes [M, K], scales [M, K/128]) outputs of a 1x128 quantizer."""
    if out is None:
        return (torch.empty((M, K), dtype=torch.uint8, device=device),
                torch.empty((M, K // 128), dtype=torch.float32, device=device))
    if len(out) != 2:
        raise ValueError("out must be a pair (codes, scales)")
    return (_out(out[0], (M, K), _CODE_DTYPES, device, "out[0]", nq),
            _out(out[1], (M, K // 128), (torch.float32,), device, "out[1]", ns))


def _same_device(device, *named):
    for name, t in named:
        if t.device != device:
            raise ValueError("%s must be on %s, got %s" % (name, device, t.device))


def _workspace(workspace, need, device):
    if workspace is None:
        return torch.empty(need, dtype=torch.uint8, device=device) if need > 0 else None
    if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on %s" % device)
    return workspace


def _y_out(out, M, N, code, device):
    dt = torch.bfloat16 if code == OUT_BF16 else torch.float32
    if out is None:
        return torch.empty((M, N), dtype=dt, device=device)
    return _out(out, (M, N), (dt,), device, "out")


# ---- quantizers ----------------------------------------------------------------

def quant_act_1x128(x: torch.Tensor, mode: int = SCALE_EXACT, out=None):
    """bf16 [M, K] -> (codes uint8 [M, K], scales fp32 [M, K/128])."""
    x = _bf16_payload(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    xq, xs = _pair_out(out, M, K, x.device)
    _check("quant_act_1x128", lib().quant_act_1x128(_ptr(x), M, K, _ptr(xq), _ptr(xs), int(mode), _stream(x)))
    return xq, xs


def quant_act_1x128_gather(x: torch.Tensor, rows: torch.Tensor, mode: int = SCALE_EXACT, out=None):
    """bf16 token rows [T, K] and int32 row indices [M] (device) -> quant_act_1x128 of
    x[rows]: (codes uint8 [M, K], scales fp32 [M, K/128])."""
    x = _bf16_payload(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [T, K]")
    if rows.dtype != torch.int32 or rows.dim() != 1 or not rows.is_contiguous() or rows.device != x.device:
        raise ValueError("rows must be a contiguous 1-D int32 tensor on x's device")
    T, K = x.shape
    M = rows.shape[0]
    xq, xs = _pair_out(out, M, K, x.device)
    _check("quant_act_1x128_gather", lib().quant_act_1x128_gather(_ptr(x), T, K, _ptr(rows), M, _ptr(xq), _ptr(xs),
                                                                 int(mode), _stream(x)))
    return xq, xs


def quant_act_1x128_scatter(x: torch.Tensor, dest: torch.Tensor, M: int, mode: int = SCALE_EXACT, out=None):
    """bf16 token rows [T, K] and int32 destinations [T, topk] (device) -> codes [M, K] and
    scales [M, K/128] where row dest[t, k] (if in [0, M)) holds quant_act_1x128 of x[t].
    Rows no destination names are left as they are: pass `out` when dest does not cover
    all M rows (the outputs allocated here start uninitialized)."""
    x = _bf16_payload(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [T, K]")
    T, K = x.shape
    if dest.dtype != torch.int32 or dest.dim() != 2 or dest.shape[0] != T or not dest.is_contiguous() or \
            dest.device != x.device:
        raise ValueError("dest must be a contiguous int32 [T, topk] tensor on x's device")
    xq, xs = _pair_out(out, int(M), K, x.device)
    _check("quant_act_1x128_scatter", lib().quant_act_1x128_scatter(_ptr(x), T, K, _ptr(dest), dest.shape[1], int(M),
                                                                   _ptr(xq), _ptr(xs), int(mode), _stream(x)))
    return xq, xs


def swiglu_quant_1x128(gu: torch.Tensor, mode: int = SCALE_EXACT, out=None):
    """bf16 gate+up output [M, 2F] (gate columns first) -> the gated activation,
    rounded to bf16 and quantized 1x128: (codes uint8 [M, F], scales fp32 [M, F/128])."""
    gu = _bf16_payload(gu, "gu")
    if gu.dim() != 2 or gu.shape[1] % 2:
        raise ValueError("gu must be 2-D [M, 2F]")
    M, F = gu.shape[0], gu.shape[1] // 2
    hq, hs = _pair_out(out, M, F, gu.device, "hq", "hs")
    _check("swiglu_quant_1x128", lib().swiglu_quant_1x128(_ptr(gu), M, F, _ptr(hq), _ptr(hs), int(mode), _stream(gu)))
    return hq, hs


def quant_act_1x128_t(x: torch.Tensor, mode: int = SCALE_EXACT, out=None):
    """bf16 [M, K] -> quant_act_1x128 of X^T: (codes uint8 [K, M], scales fp32 [K, M/128])."""
    x = _bf16_payload(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    xqt, xst = _pair_out(out, K, M, x.device, "xqt", "xst")
    _check("quant_act_1x128_t", lib().quant_act_1x128_t(_ptr(x), M, K, _ptr(xqt), _ptr(xst), int(mode), _stream(x)))
    return xqt, xst


def quant_act_1x128_dual(x: torch.Tensor, mode: int = SCALE_EXACT, out=None):
    """bf16 [M, K] -> (xq [M, K], xs [M, K/128], xqt [K, M], xst [K, M/128]): quant_act_1x128
    of X and of X^T from one read of X."""
    x = _bf16_payload(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    if out is not None and len(out) != 4:
        raise ValueError("out must be (xq, xs, xqt, xst)")
    xq, xs = _pair_out(None if out is None else out[:2], M, K, x.device)
    xqt, xst = _pair_out(None if out is None else out[2:], K, M, x.device, "xqt", "xst")
    _check("quant_act_1x128_dual", lib().quant_act_1x128_dual(_ptr(x), M, K, _ptr(xq), _ptr(xs), _ptr(xqt),
                                                              _ptr(xst), int(mode), _stream(x)))
    return xq, xs, xqt, xst


def quant_w_128x128(w: torch.Tensor, mode: int = SCALE_EXACT, out=None):
    """bf16 [N, K] -> (codes uint8 [N, K], scales fp32 [N/128, K/128])."""
    w = _bf16_payload(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    N, K = w.shape
    wq, ws = _w_out(out, w)
    _check("quant_w_128x128", lib().quant_w_128x128(_ptr(w), N, K, _ptr(wq), _ptr(ws), int(mode), _stream(w)))
    return wq, ws


def quant_w_128x128_batched(ws_in: Sequence[torch.Tensor], mode: int = SCALE_EXACT, outs=None):
    """Re-quantize many weight tensors in one call (per-step recalibration)."""
    n = len(ws_in)
    if n == 0:
        return []
    tensors = [_bf16_payload(w, "w[%d]" % i) for i, w in enumerate(ws_in)]
    _batch_devices(tensors)
    if outs is not None and len(outs) != n:
        raise ValueError("outs must hold one (codes, scales) pair per weight")
    outs = [_w_out(None if outs is None else outs[i], w) for i, w in enumerate(tensors)]
    arr_p = ctypes.c_void_p * n
    arr_i = ctypes.c_int64 * n
    wp = arr_p(*[w.data_ptr() for w in tensors])
    Ns = arr_i(*[w.shape[0] for w in tensors])
    Ks = arr_i(*[w.shape[1] for w in tensors])
    qp = arr_p(*[o[0].data_ptr() for o in outs])
    sp = arr_p(*[o[1].data_ptr() for o in outs])
    st = lib().quant_w_128x128_batched(n, ctypes.cast(wp, ctypes.c_void_p), ctypes.cast(Ns, ctypes.c_void_p),
                                       ctypes.cast(Ks, ctypes.c_void_p), ctypes.cast(qp, ctypes.c_void_p),
                                       ctypes.cast(sp, ctypes.c_void_p), int(mode), _stream(tensors[0]))
    _check("quant_w_128x128_batched", st)
    return outs


def _w_out(out, w: torch.Tensor):
    """(codes [N, K], scales [N/128, K/128]) outputs of the 128x128 quantizer."""
    N, K = w.shape
    if out is None:
        return (torch.empty((N, K), dtype=torch.uint8, device=w.device),
                torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device))
    if len(out) != 2:
        raise ValueError("out must be a pair (codes, scales)")
    return (_out(out[0], (N, K), _CODE_DTYPES, w.device, "out[0] (wq)"),
            _out(out[1], (N // 128, K // 128), (torch.float32,), w.device, "out[1] (ws)"))


def _batch_devices(tensors):
    for i, w in enumerate(tensors):
        if w.dim() != 2:
            raise ValueError("w[%d] must be 2-D [N, K]" % i)
        _same_device(tensors[0].device, ("w[%d]" % i, w))


def _dual_outs(w: torch.Tensor, out=None):
    """(wq [N, K], ws [N/128, K/128], wqt [K, N], wst [K/128, N/128]) of the dual quantizer."""
    N, K = w.shape
    if out is not None and len(out) != 4:
        raise ValueError("out must be (wq, ws, wqt, wst)")
    wq, ws = _w_out(None if out is None else out[:2], w)
    if out is None:
        return (wq, ws, torch.empty((K, N), dtype=torch.uint8, device=w.device),
                torch.empty((K // 128, N // 128), dtype=torch.float32, device=w.device))
    return (wq, ws, _out(out[2], (K, N), _CODE_DTYPES, w.device, "out[2] (wqt)"),
            _out(out[3], (K // 128, N // 128), (torch.float32,), w.device, "out[3] (wst)"))


def quant_w_128x128_dual(w: torch.Tensor, mode: int = SCALE_EXACT, out=None):
    """bf16 [N, K] -> (wq [N, K], ws [N/128, K/128], wqt [K, N], wst [K/128, N/128]):
    the codes and scales of W and of W^T from one read of W."""
    w = _bf16_payload(w, "w")
    if w.dim() != 2:
        raise ValueError("w must be 2-D [N, K]")
    N, K = w.shape
    wq, ws, wqt, wst = _dual_outs(w, out)
    _check("quant_w_128x128_dual", lib().quant_w_128x128_dual(_ptr(w), N, K, _ptr(wq), _ptr(ws), _ptr(wqt),
                                                              _ptr(wst), int(mode), _stream(w)))
    return wq, ws, wqt, wst


def quant_w_128x128_dual_batched(ws_in: Sequence[torch.Tensor], mode: int = SCALE_EXACT, outs=None):
    """quant_w_128x128_dual over many weight tensors in one call."""
    n = len(ws_in)
    if n == 0:
        return []
    tensors = [_bf16_payload(w, "w[%d]" % i) for i, w in enumerate(ws_in)]
    _batch_devices(tensors)
    if outs is not None and len(outs) != n:
        raise ValueError("outs must hold one (wq, ws, wqt, wst) tuple per weight")
    outs = [_dual_outs(w, None if outs is None else outs[i]) for i, w in enumerate(tensors)]
    arr_p = ctypes.c_void_p * n
    arr_i = ctypes.c_int64 * n
    cols = [arr_p(*[o[j].data_ptr() for o in outs]) for j in range(4)]
    wp = arr_p(*[w.data_ptr() for w in tensors])
    Ns = arr_i(*[w.shape[0] for w in tensors])
    Ks = arr_i(*[w.shape[1] for w in tensors])
    cv = lambda a: ctypes.cast(a, ctypes.c_void_p)  # noqa: E731
    st = lib().quant_w_128x128_dual_batched(n, cv(wp), cv(Ns), cv(Ks), *[cv(c) for c in cols], int(mode),
                                            _stream(tensors[0]))
    _check("quant_w_128x128_dual_batched", st)
    return outs


# ---- GEMMs ---------------------------------------------------------------------

def _out_code(out_dtype) -> int:
    if out_dtype in (torch.bfloat16, OUT_BF16):
        return OUT_BF16
    if out_dtype in (torch.float32, OUT_FP32):
        return OUT_FP32
    raise ValueError("out_dtype must be torch.bfloat16 or torch.float32")


def gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().fp8bs_gemm_workspace_size(M, N, K))


def grouped_workspace_size(E: int, M_total: int, N: int, K: int) -> int:
    return int(lib().fp8bs_grouped_workspace_size(E, M_total, N, K))


def fp8_block_gemm(xq, xs, wq, ws, out_dtype=torch.bfloat16, out=None, workspace=None):
    """Y [M, N] = dequant(xq, xs) @ dequant(wq, ws)^T."""
    return _gemm("fp8_block_gemm", xq, xs, wq, ws, out_dtype, out, workspace)


def fp8_block_gemm_pow2(xq, xs, wq, ws, out_dtype=torch.bfloat16, out=None, workspace=None):
    """fp8_block_gemm for power-of-2 scales (POW2-quantized operands): the scales go to the matrix cores."""
    return _gemm("fp8_block_gemm_pow2", xq, xs, wq, ws, out_dtype, out, workspace)


def fp8_block_gemm_1x128(xq, xs, wq, ws, out_dtype=torch.bfloat16, out=None):
    """Y [M, N] with 1x128 scales on both operands (ws [N, K/128]): the weight gradient
    dW = dY^T X from quant_act_1x128_t(dY) and quant_act_1x128_t(X)."""
    return _gemm_1x128("fp8_block_gemm_1x128", xq, xs, wq, ws, out_dtype, out)


def fp8_block_gemm_1x128_pow2(xq, xs, wq, ws, out_dtype=torch.bfloat16, out=None):
    """fp8_block_gemm_1x128 for operands quantized with power-of-2 scales (both scales go to the
    matrix cores)."""
    return _gemm_1x128("fp8_block_gemm_1x128_pow2", xq, xs, wq, ws, out_dtype, out)


def _gemm_1x128(fn, xq, xs, wq, ws, out_dtype, out):
    xq, wq = _codes(xq, "xq"), _codes(wq, "wq")
    xs, ws = _f32(xs, "xs"), _f32(ws, "ws")
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or xs.shape != (M, K // 128) or ws.shape != (N, K // 128):
        raise ValueError("operand shapes do not match")
    _same_device(xq.device, ("xs", xs), ("wq", wq), ("ws", ws))
    code = _out_code(out_dtype)
    out = _y_out(out, M, N, code, xq.device)
    _check(fn, getattr(lib(), fn)(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(out), code, _stream(xq)))
    return out


def _gemm(fn, xq, xs, wq, ws, out_dtype, out, workspace):
    xq, wq = _codes(xq, "xq"), _codes(wq, "wq")
    xs, ws = _f32(xs, "xs"), _f32(ws, "ws")
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or xs.shape != (M, K // 128) or ws.shape != (N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    _same_device(xq.device, ("xs", xs), ("wq", wq), ("ws", ws))
    code = _out_code(out_dtype)
    out = _y_out(out, M, N, code, xq.device)
    workspace = _workspace(workspace, gemm_workspace_size(M, N, K), xq.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = getattr(lib(), fn)(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(out), code,
                            _ptr(workspace), wsz, _stream(xq))
    _check(fn, st)
    return out


def gemm_quant_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().fp8bs_gemm_quant_workspace_size(M, N, K))


def fp8_block_gemm_quant(xq, xs, wq, ws, mode: int = SCALE_EXACT, want_y: bool = True, out=None, workspace=None):
    """(y bf16 [M, N] or None, yq codes [M, N], ys scales [M, N/128]): the GEMM and
    quant_act_1x128 of its bf16 output from one call (fused into the GEMM's epilogue
    where the shape allows).  `mode` is the scale mode of the operands and the output."""
    xq, wq = _codes(xq, "xq"), _codes(wq, "wq")
    xs, ws = _f32(xs, "xs"), _f32(ws, "ws")
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or xs.shape != (M, K // 128) or ws.shape != (N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    _same_device(xq.device, ("xs", xs), ("wq", wq), ("ws", ws))
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be (y or None, yq, ys)")
        y = None if out[0] is None else _y_out(out[0], M, N, OUT_BF16, xq.device)
        yq, ys = _pair_out(out[1:], M, N, xq.device, "yq", "ys")
    else:
        y = _y_out(None, M, N, OUT_BF16, xq.device) if want_y else None
        yq, ys = _pair_out(None, M, N, xq.device, "yq", "ys")
    workspace = _workspace(workspace, gemm_quant_workspace_size(M, N, K), xq.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fp8_block_gemm_quant(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), M, N, K, _ptr(y), _ptr(yq), _ptr(ys),
                                    int(mode), _ptr(workspace), wsz, _stream(xq))
    _check("fp8_block_gemm_quant", st)
    return y, yq, ys


def linear_workspace_size(M: int, N: int, K: int) -> int:
    return int(lib().fp8bs_linear_workspace_size(M, N, K))


def fp8_block_linear(x, wq, ws, out_dtype=torch.bfloat16, out=None, workspace=None):
    """Y [M, N] = fp8_block_gemm(quant_act_1x128(x), wq, ws) from bf16 x [M, K] (one launch for decode rows)."""
    return _linear("fp8_block_linear", x, wq, ws, out_dtype, out, workspace)


def fp8_block_linear_pow2(x, wq, ws, out_dtype=torch.bfloat16, out=None, workspace=None):
    """fp8_block_linear with x quantized to power-of-2 scales (ws must hold POW2 scales)."""
    return _linear("fp8_block_linear_pow2", x, wq, ws, out_dtype, out, workspace)


def _linear(fn, x, wq, ws, out_dtype, out, workspace):
    x = _bf16_payload(x, "x")
    wq, ws = _codes(wq, "wq"), _f32(ws, "ws")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = x.shape
    N = wq.shape[0]
    if wq.shape[1] != K or ws.shape != (N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    _same_device(x.device, ("wq", wq), ("ws", ws))
    code = _out_code(out_dtype)
    out = _y_out(out, M, N, code, x.device)
    workspace = _workspace(workspace, linear_workspace_size(M, N, K), x.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = getattr(lib(), fn)(_ptr(x), _ptr(wq), _ptr(ws), M, N, K, _ptr(out), code, _ptr(workspace), wsz, _stream(x))
    _check(fn, st)
    return out


def fp8_block_grouped_gemm(xq, xs, wq, ws, group_offsets, out_dtype=torch.bfloat16, out=None, workspace=None):
    """Y [M_total, N]: rows offs[e]..offs[e+1]-1 multiplied by expert e's weights."""
    return _grouped("fp8_block_grouped_gemm", xq, xs, wq, ws, group_offsets, out_dtype, out, workspace)


def fp8_block_grouped_gemm_pow2(xq, xs, wq, ws, group_offsets, out_dtype=torch.bfloat16, out=None, workspace=None):
    """fp8_block_grouped_gemm for power-of-2 scales (POW2-quantized operands)."""
    return _grouped("fp8_block_grouped_gemm_pow2", xq, xs, wq, ws, group_offsets, out_dtype, out, workspace)


def fp8_block_grouped_gemm_noalloc(xq, xs, wq, ws, group_offsets, out_dtype=torch.bfloat16, out=None):
    """fp8_block_grouped_gemm whose library call allocates nothing: its row-tile tables live in
    the library's static device array (calls overlapping in time on one GPU race on it).  Pass
    `out` to keep this call free of allocations on the Python side too."""
    return _grouped("fp8_block_grouped_gemm_noalloc", xq, xs, wq, ws, group_offsets, out_dtype, out, None,
                    noalloc=True)


def _grouped(fn, xq, xs, wq, ws, group_offsets, out_dtype, out, workspace, noalloc=False):
    xq, wq = _codes(xq, "xq"), _codes(wq, "wq")
    xs, ws = _f32(xs, "xs"), _f32(ws, "ws")
    if group_offsets.dtype != torch.int32 or not group_offsets.is_cuda or not group_offsets.is_contiguous():
        raise ValueError("group_offsets must be a contiguous int32 device tensor")
    if xq.dim() != 2 or wq.dim() != 3:
        raise ValueError("xq must be [M_total, K] and wq [E, N, K]")
    M, K = xq.shape
    E, N, K2 = wq.shape
    if K2 != K or xs.shape != (M, K // 128) or ws.shape != (E, N // 128, K // 128) or group_offsets.numel() != E + 1:
        raise ValueError("operand shapes do not match")
    _same_device(xq.device, ("xs", xs), ("wq", wq), ("ws", ws), ("group_offsets", group_offsets))
    code = _out_code(out_dtype)
    out = _y_out(out, M, N, code, xq.device)
    if noalloc:
        st = getattr(lib(), fn)(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(group_offsets), E, M, N, K,
                                _ptr(out), code, _stream(xq))
        _check(fn, st)
        return out
    workspace = _workspace(workspace, grouped_workspace_size(E, M, N, K), xq.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = getattr(lib(), fn)(_ptr(xq), _ptr(xs), _ptr(wq), _ptr(ws), _ptr(group_offsets), E, M, N, K,
                            _ptr(out), code, _ptr(workspace), wsz, _stream(xq))
    _check(fn, st)
    return out


# ---- attention over an FP8 KV cache ---------------------------------------------

def kv_attention_workspace_size(B: int, T: int, Hq: int, Hkv: int) -> int:
    return int(lib().fp8bs_kv_attention_workspace_size(B, T, Hq, Hkv))


def fp8_kv_attention_decode(q, kq, ks, vq, vs, lens, sm_scale: float, out_dtype=torch.bfloat16, out=None,
                            workspace=None):
    """o [B, Hq, 128]: each sequence's new query token q [B, Hq, 128] (bf16) attending to
    its first lens[b] cached tokens; kq, vq [B, T, Hkv, 128] codes and ks, vs [B, T, Hkv]
    scales (quant_act_1x128 of the key / value rows); lens int32 [B] on the device."""
    q = _bf16_payload(q, "q")
    kq, vq = _codes(kq, "kq"), _codes(vq, "vq")
    ks, vs = _f32(ks, "ks"), _f32(vs, "vs")
    if q.dim() != 3 or kq.dim() != 4 or q.shape[2] != 128 or kq.shape[3] != 128:
        raise ValueError("q must be [B, Hq, 128] and kq [B, T, Hkv, 128]")
    B, Hq, _ = q.shape
    _, T, Hkv, _ = kq.shape
    if kq.shape[0] != B or vq.shape != kq.shape or ks.shape != (B, T, Hkv) or vs.shape != ks.shape:
        raise ValueError("cache shapes do not match")
    if lens.dtype != torch.int32 or tuple(lens.shape) != (B,) or not lens.is_contiguous():
        raise ValueError("lens must be a contiguous int32 [B] tensor")
    _same_device(q.device, ("kq", kq), ("ks", ks), ("vq", vq), ("vs", vs), ("lens", lens))
    code = _out_code(out_dtype)
    dt = torch.bfloat16 if code == OUT_BF16 else torch.float32
    out = torch.empty((B, Hq, 128), dtype=dt, device=q.device) if out is None else \
        _out(out, (B, Hq, 128), (dt,), q.device, "out")
    workspace = _workspace(workspace, kv_attention_workspace_size(B, T, Hq, Hkv), q.device)
    wsz = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fp8_kv_attention_decode(_ptr(q), _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs), _ptr(lens), B, T, Hq, Hkv,
                                       float(sm_scale), _ptr(out), code, _ptr(workspace), wsz, _stream(q))
    _check("fp8_kv_attention_decode", st)
    return out
