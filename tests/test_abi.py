"""The C-ABI library: it loads, exports every function include/fp8bs.h declares,
and rejects bad arguments before touching a device.

These run on any host: every call below fails validation (or is a pure query)
before the library makes a HIP call, except the device-check test, which only
asks the runtime which device is current and is skipped when a GPU is present.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8bs.h")


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    if not os.path.exists(m.LIB_PATH):
        from block_scaled_fp8_x128_amd import build
        build.build()
    return m


def _declared_functions():
    text = open(HEADER).read()
    return re.findall(r"^FP8BS_API\s+(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def test_header_declares_the_boundary():
    names = _declared_functions()
    for fn in ("quant_act_1x128", "quant_w_128x128", "fp8_block_gemm", "fp8_block_grouped_gemm"):
        assert fn in names


def test_library_exports_every_declared_symbol(fp8bs):
    L = fp8bs.lib()
    names = _declared_functions()
    assert set(names) == set(fp8bs.EXPORTS)
    for fn in names:
        assert hasattr(L, fn), fn
    # and nothing else: internal C++ symbols stay hidden
    out = os.popen("nm -D --defined-only %s" % fp8bs.LIB_PATH).read()
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    assert exported == set(names)


def test_version_and_status_strings(fp8bs):
    assert fp8bs.abi_version() == 2
    for st in range(7):
        s = fp8bs.status_string(st)
        assert isinstance(s, str) and len(s) > 1
    assert fp8bs.status_string(99) == "unknown status"


def test_workspace_queries_are_pure(fp8bs):
    L = fp8bs.lib()
    assert L.fp8bs_gemm_workspace_size(0, 128, 128) == 0
    assert L.fp8bs_gemm_workspace_size(-1, 128, 128) == 0
    # grouped: 16 bytes of tile counts, then two row-tile tables of 16-byte entries: the 256-row
    # tiles (at most ceil(M_total / 256) + E) and the experts' short last tiles (at most E)
    assert L.fp8bs_grouped_workspace_size(128, 65536, 1536, 2048) == 16 + 16 * (65536 // 256 + 128 + 128)
    assert L.fp8bs_grouped_workspace_size(0, 65536, 1536, 2048) == 0
    # dense: fp32 partial sums (ksplit slices of M x N) when the product is split along K,
    # never for products with at least one 256 x 256 tile per compute unit
    assert L.fp8bs_gemm_workspace_size(8192, 28672, 4096) == 0
    assert L.fp8bs_gemm_workspace_size(8192, 4096, 14336) == 0
    for M, N, K in ((64, 4096, 14336), (256, 4096, 14336), (40, 512, 8192)):
        ws = L.fp8bs_gemm_workspace_size(M, N, K)
        assert ws > 0 and ws % (M * N * 4) == 0 and 2 <= ws // (M * N * 4) <= K // 128


FAKE = ctypes.c_void_p(0x10000)      # never dereferenced: validation fails first
MISAL = ctypes.c_void_p(0x10008)     # 8-byte aligned only
NULL = ctypes.c_void_p(0)


def test_quant_act_validation(fp8bs):
    L = fp8bs.lib()
    q = L.quant_act_1x128
    assert q(FAKE, 4, 100, FAKE, FAKE, 0, NULL) == 2      # K % 128
    assert q(FAKE, -1, 128, FAKE, FAKE, 0, NULL) == 1     # negative M
    assert q(FAKE, 4, 0, FAKE, FAKE, 0, NULL) == 1        # K == 0
    assert q(FAKE, 4, 128, FAKE, FAKE, 7, NULL) == 1      # unknown mode
    assert q(NULL, 4, 128, FAKE, FAKE, 0, NULL) == 1      # null input
    assert q(FAKE, 4, 128, NULL, FAKE, 0, NULL) == 1      # null codes
    assert q(FAKE, 4, 128, FAKE, NULL, 0, NULL) == 1      # null scales
    assert q(MISAL, 4, 128, FAKE, FAKE, 0, NULL) == 1     # misaligned input
    assert q(NULL, 0, 128, NULL, NULL, 0, NULL) == 0      # M == 0: no-op


def test_quant_act_gather_validation(fp8bs):
    L = fp8bs.lib()
    q = L.quant_act_1x128_gather
    assert q(FAKE, 8, 100, FAKE, 4, FAKE, FAKE, 0, NULL) == 2       # K % 128
    assert q(FAKE, 8, 1 << 14, FAKE, 1 << 24, FAKE, FAKE, 0, NULL) == 2   # 2^31 blocks
    assert q(FAKE, -1, 128, FAKE, 4, FAKE, FAKE, 0, NULL) == 1      # negative T
    assert q(FAKE, 8, 128, FAKE, -1, FAKE, FAKE, 0, NULL) == 1      # negative M
    assert q(FAKE, 8, 0, FAKE, 4, FAKE, FAKE, 0, NULL) == 1         # K == 0
    assert q(FAKE, 8, 128, FAKE, 4, FAKE, FAKE, 2, NULL) == 1       # unknown mode
    assert q(NULL, 8, 128, FAKE, 4, FAKE, FAKE, 0, NULL) == 1       # null input
    assert q(FAKE, 8, 128, NULL, 4, FAKE, FAKE, 0, NULL) == 1       # null rows
    assert q(FAKE, 8, 128, FAKE, 4, NULL, FAKE, 0, NULL) == 1       # null codes
    assert q(FAKE, 8, 128, FAKE, 4, FAKE, NULL, 0, NULL) == 1       # null scales
    assert q(MISAL, 8, 128, FAKE, 4, FAKE, FAKE, 0, NULL) == 1      # misaligned input
    assert q(NULL, 0, 128, NULL, 0, NULL, NULL, 0, NULL) == 0       # M == 0: no-op


def test_swiglu_quant_validation(fp8bs):
    L = fp8bs.lib()
    q = L.swiglu_quant_1x128
    assert q(FAKE, 4, 100, FAKE, FAKE, 0, NULL) == 2      # F % 128
    assert q(FAKE, 1 << 24, 1 << 14, FAKE, FAKE, 0, NULL) == 2   # 2^31 blocks
    assert q(FAKE, -1, 128, FAKE, FAKE, 0, NULL) == 1     # negative M
    assert q(FAKE, 4, 0, FAKE, FAKE, 0, NULL) == 1        # F == 0
    assert q(FAKE, 4, 128, FAKE, FAKE, 2, NULL) == 1      # unknown mode
    assert q(NULL, 4, 128, FAKE, FAKE, 0, NULL) == 1      # null input
    assert q(FAKE, 4, 128, NULL, FAKE, 0, NULL) == 1      # null codes
    assert q(FAKE, 4, 128, FAKE, NULL, 0, NULL) == 1      # null scales
    assert q(MISAL, 4, 128, FAKE, FAKE, 0, NULL) == 1     # misaligned input
    assert q(FAKE, 4, 128, MISAL, FAKE, 0, NULL) == 1     # misaligned codes
    assert q(NULL, 0, 128, NULL, NULL, 0, NULL) == 0      # M == 0: no-op


def test_quant_w_validation(fp8bs):
    L = fp8bs.lib()
    q = L.quant_w_128x128
    assert q(FAKE, 100, 128, FAKE, FAKE, 0, NULL) == 2     # N % 128
    assert q(FAKE, 128, 130, FAKE, FAKE, 0, NULL) == 2     # K % 128
    assert q(FAKE, 128, 128, FAKE, FAKE, -1, NULL) == 1
    assert q(NULL, 0, 128, NULL, NULL, 1, NULL) == 0
    b = L.quant_w_128x128_batched
    assert b(-1, NULL, NULL, NULL, NULL, NULL, 0, NULL) == 1
    assert b(0, NULL, NULL, NULL, NULL, NULL, 0, NULL) == 0
    assert b(2, NULL, NULL, NULL, NULL, NULL, 0, NULL) == 1
    arr = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    Ns = (ctypes.c_int64 * 2)(128, 100)
    Ks = (ctypes.c_int64 * 2)(128, 128)
    assert b(2, arr, Ns, Ks, arr, arr, 0, NULL) == 2      # second tensor N % 128


def test_quant_w_dual_validation(fp8bs):
    L = fp8bs.lib()
    q = L.quant_w_128x128_dual
    assert q(FAKE, 100, 128, FAKE, FAKE, FAKE, FAKE, 0, NULL) == 2     # N % 128
    assert q(FAKE, 128, 130, FAKE, FAKE, FAKE, FAKE, 0, NULL) == 2     # K % 128
    assert q(FAKE, 128, 128, FAKE, FAKE, FAKE, FAKE, 2, NULL) == 1     # unknown mode
    assert q(FAKE, 128, 128, FAKE, FAKE, NULL, FAKE, 0, NULL) == 1     # null transposed codes
    assert q(FAKE, 128, 128, FAKE, FAKE, FAKE, NULL, 0, NULL) == 1     # null transposed scales
    assert q(FAKE, 128, 128, FAKE, FAKE, MISAL, FAKE, 0, NULL) == 1    # misaligned transposed codes
    assert q(FAKE, 128, 128, NULL, FAKE, FAKE, FAKE, 0, NULL) == 1     # null codes
    assert q(NULL, 0, 128, NULL, NULL, NULL, NULL, 1, NULL) == 0       # N == 0: no-op
    b = L.quant_w_128x128_dual_batched
    assert b(-1, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == 1
    assert b(0, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL) == 0
    arr = (ctypes.c_void_p * 2)(0x10000, 0x20000)
    Ns = (ctypes.c_int64 * 2)(128, 128)
    Ks = (ctypes.c_int64 * 2)(128, 128)
    assert b(2, arr, Ns, Ks, arr, arr, NULL, arr, 0, NULL) == 1        # null transposed-codes array
    bad = (ctypes.c_void_p * 2)(0x10000, 0x20008)
    assert b(2, arr, Ns, Ks, arr, arr, bad, arr, 0, NULL) == 1         # second tensor misaligned


def test_weight_gradient_entry_validation(fp8bs):
    L = fp8bs.lib()
    q = L.quant_act_1x128_t
    assert q(FAKE, 100, 128, FAKE, FAKE, 0, NULL) == 2     # M % 128 (blocks run down the columns)
    assert q(FAKE, 128, 100, FAKE, FAKE, 0, NULL) == 2     # K % 128
    assert q(FAKE, 128, 128, FAKE, FAKE, 3, NULL) == 1     # unknown mode
    assert q(FAKE, 128, 128, NULL, FAKE, 0, NULL) == 1     # null codes
    assert q(MISAL, 128, 128, FAKE, FAKE, 0, NULL) == 1    # misaligned input
    assert q(NULL, 0, 128, NULL, NULL, 0, NULL) == 0       # M == 0: no-op
    d = L.quant_act_1x128_dual
    assert d(FAKE, 100, 128, FAKE, FAKE, FAKE, FAKE, 0, NULL) == 2     # M % 128
    assert d(FAKE, 128, 128, FAKE, FAKE, NULL, FAKE, 0, NULL) == 1     # null transposed codes
    assert d(FAKE, 128, 128, NULL, FAKE, FAKE, FAKE, 0, NULL) == 1     # null row codes
    assert d(FAKE, 128, 128, FAKE, FAKE, MISAL, FAKE, 0, NULL) == 1    # misaligned transposed codes
    assert d(NULL, 0, 128, NULL, NULL, NULL, NULL, 1, NULL) == 0       # M == 0: no-op
    g = L.fp8_block_gemm_1x128
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 100, 128, FAKE, 0, NULL) == 2   # N % 128
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 128, 100, FAKE, 0, NULL) == 2   # K % 128
    assert g(FAKE, FAKE, FAKE, FAKE, -1, 128, 128, FAKE, 0, NULL) == 1  # M < 0
    assert g(FAKE, FAKE, FAKE, NULL, 8, 128, 128, FAKE, 0, NULL) == 1   # null weight scales
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 128, 128, MISAL, 0, NULL) == 1  # misaligned output
    assert g(NULL, NULL, FAKE, FAKE, 0, 128, 128, NULL, 0, NULL) == 0   # M == 0: no-op


def test_gemm_validation(fp8bs):
    L = fp8bs.lib()
    g = L.fp8_block_gemm
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 100, 128, FAKE, 0, NULL, 0, NULL) == 2   # N % 128
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 128, 100, FAKE, 0, NULL, 0, NULL) == 2   # K % 128
    assert g(FAKE, FAKE, FAKE, FAKE, -8, 128, 128, FAKE, 0, NULL, 0, NULL) == 1  # M < 0
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 128, 128, FAKE, 5, NULL, 0, NULL) == 1   # out dtype
    assert g(FAKE, FAKE, NULL, FAKE, 8, 128, 128, FAKE, 0, NULL, 0, NULL) == 1   # null weights
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 128, 128, NULL, 0, NULL, 0, NULL) == 1   # null output
    assert g(FAKE, FAKE, FAKE, FAKE, 8, 128, 128, MISAL, 0, NULL, 0, NULL) == 1  # misaligned output
    assert g(FAKE, FAKE, FAKE, FAKE, 2**30, 2**30, 128, FAKE, 0, NULL, 0, NULL) == 2  # 2^36 output tiles
    assert g(NULL, NULL, FAKE, FAKE, 0, 128, 128, NULL, 0, NULL, 0, NULL) == 0   # M == 0
    need = L.fp8bs_gemm_workspace_size(64, 4096, 14336)
    assert g(FAKE, FAKE, FAKE, FAKE, 64, 4096, 14336, FAKE, 0, NULL, 0, NULL) == 4          # no workspace
    assert g(FAKE, FAKE, FAKE, FAKE, 64, 4096, 14336, FAKE, 0, FAKE, need - 1, NULL) == 4   # too small
    assert g(FAKE, FAKE, FAKE, FAKE, 64, 4096, 14336, FAKE, 0, MISAL, need, NULL) == 1      # misaligned
    gg = L.fp8_block_grouped_gemm
    assert gg(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 128, FAKE, 0, NULL, 0, NULL) == 1   # E == 0
    assert gg(FAKE, FAKE, FAKE, FAKE, NULL, 4, 8, 128, 128, FAKE, 0, NULL, 0, NULL) == 1   # null offsets
    assert gg(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 96, 128, FAKE, 0, NULL, 0, NULL) == 2    # N % 128
    assert gg(NULL, NULL, FAKE, FAKE, FAKE, 4, 0, 128, 128, NULL, 0, NULL, 0, NULL) == 0   # empty
    assert gg(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 256, 256, FAKE, 0, NULL, 0, NULL) == 4   # no table space


def test_gemm_quant_workspace_and_validation(fp8bs):
    """fp8_block_gemm_quant: no workspace where the quantization runs in the 256x256 kernel's
    epilogue (at least one 256x256 tile per compute unit); elsewhere a bf16 Y buffer (16-byte
    aligned) followed by fp8_block_gemm's workspace.  y may be NULL; yq and ys may not."""
    L = fp8bs.lib()
    wsz = L.fp8bs_gemm_quant_workspace_size
    for M, N, K in ((8192, 4096, 4096), (8192, 28672, 4096), (8200, 8192, 1024)):
        assert wsz(M, N, K) == 0
    for M, N, K in ((300, 512, 1024), (1, 256, 2048), (64, 4096, 14336)):
        assert wsz(M, N, K) == (M * N * 2 + 15) // 16 * 16 + L.fp8bs_gemm_workspace_size(M, N, K)
    assert wsz(0, 128, 128) == 0
    g = L.fp8_block_gemm_quant
    F = FAKE
    assert g(F, F, F, F, 8, 128, 128, F, F, F, 2, NULL, 0, NULL) == 1        # scale mode
    assert g(F, F, F, F, 8, 100, 128, F, F, F, 0, NULL, 0, NULL) == 2        # N % 128
    assert g(F, F, F, F, -8, 128, 128, F, F, F, 0, NULL, 0, NULL) == 1       # M < 0
    assert g(F, F, F, F, 8, 128, 128, F, NULL, F, 0, NULL, 0, NULL) == 1     # null codes out
    assert g(F, F, F, F, 8, 128, 128, F, F, NULL, 0, NULL, 0, NULL) == 1     # null scales out
    assert g(F, F, F, F, 8, 128, 128, MISAL, F, F, 0, NULL, 0, NULL) == 1    # misaligned y
    assert g(F, F, F, F, 8, 128, 128, F, MISAL, F, 0, NULL, 0, NULL) == 1    # misaligned codes
    assert g(NULL, NULL, F, F, 0, 128, 128, NULL, NULL, NULL, 1, NULL, 0, NULL) == 0   # M == 0
    need = wsz(300, 512, 1024)
    assert g(F, F, F, F, 300, 512, 1024, NULL, F, F, 0, NULL, 0, NULL) == 4            # no workspace
    assert g(F, F, F, F, 300, 512, 1024, NULL, F, F, 0, F, need - 1, NULL) == 4       # too small
    assert g(F, F, F, F, 300, 512, 1024, NULL, F, F, 0, MISAL, need, NULL) == 1       # misaligned


def test_kv_attention_workspace_and_validation(fp8bs):
    """fp8_kv_attention_decode: group sizes 1, 2, 4, 8; per-split partial states (2 + 128 fp32 per
    sequence, query head and split) when a sequence's tokens are split; argument checks."""
    L = fp8bs.lib()
    wsz = L.fp8bs_kv_attention_workspace_size
    assert wsz(4, 1024, 32, 8) % (4 * 32 * 130 * 4) == 0
    assert wsz(64, 4096, 32, 8) == 0 or wsz(64, 4096, 32, 8) % (64 * 32 * 130 * 4) == 0
    assert wsz(8, 4096, 32, 8) > 0            # 64 key/value heads: split to fill the chip
    assert wsz(1, 64, 32, 8) == 0             # one 64-token chunk: not split
    assert wsz(2, 100, 12, 8) == 0            # unsupported group: no workspace
    f = L.fp8_kv_attention_decode
    F = FAKE
    args = lambda B, T, Hq, Hkv, sm=0.1, od=0: (F, F, F, F, F, F, B, T, Hq, Hkv, ctypes.c_float(sm), F, od,  # noqa
                                                F, 1 << 30, NULL)
    assert f(*args(2, 100, 12, 8)) == 2                  # Hq / Hkv not an integer
    assert f(*args(2, 100, 48, 4)) == 2                  # group of 12
    assert f(*args(2, 100, 32, 2)) == 2                  # group of 16
    assert f(*args(-1, 100, 32, 8)) == 1                 # B < 0
    assert f(*args(2, 0, 32, 8)) == 1                    # T == 0
    assert f(*args(2, 100, 32, 8, od=4)) == 1            # out dtype
    assert f(*args(2, 100, 32, 8, sm=float("nan"))) == 1  # sm_scale
    assert f(*args(2, 1 << 22, 32, 8)) == 2              # 32-bit cache offsets
    assert f(*args(0, 100, 32, 8)) == 0                  # B == 0: no-op
    assert f(F, F, F, F, F, NULL, 2, 100, 32, 8, ctypes.c_float(0.1), F, 0, F, 1 << 30, NULL) == 1  # lens
    assert f(F, F, F, F, F, F, 2, 100, 32, 8, ctypes.c_float(0.1), MISAL, 0, F, 1 << 30, NULL) == 1  # out
    need = wsz(8, 4096, 32, 8)
    assert f(F, F, F, F, F, F, 8, 4096, 32, 8, ctypes.c_float(0.1), F, 0, F, need - 1, NULL) == 4


def test_grouped_noalloc_validation(fp8bs):
    """fp8_block_grouped_gemm_noalloc: the grouped GEMM's checks, no workspace argument, and
    SCRATCH_TOO_SMALL (before any device call) when its row-tile tables exceed the library's
    static array: 16 + 16 (ceil(M_total / 256) + 2 E) bytes against 1 MiB."""
    L = fp8bs.lib()
    gn = L.fp8_block_grouped_gemm_noalloc
    cap = fp8bs.NOALLOC_SCRATCH_BYTES
    assert gn(FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 128, 128, FAKE, 0, NULL) == 1     # E == 0
    assert gn(FAKE, FAKE, FAKE, FAKE, NULL, 4, 8, 128, 128, FAKE, 0, NULL) == 1     # null offsets
    assert gn(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 96, 128, FAKE, 0, NULL) == 2      # N % 128
    assert gn(FAKE, FAKE, FAKE, FAKE, FAKE, 4, 8, 256, 256, FAKE, 7, NULL) == 1     # out dtype
    assert gn(NULL, NULL, FAKE, FAKE, FAKE, 4, 0, 256, 256, NULL, 0, NULL) == 0     # empty: no-op
    # the largest M_total that fits with E experts, and one 256-row tile more
    for E in (1, 128):
        m_fit = ((cap - 16) // 16 - 2 * E) * 256
        assert L.fp8bs_grouped_workspace_size(E, m_fit, 256, 256) <= cap
        assert L.fp8bs_grouped_workspace_size(E, m_fit + 1, 256, 256) > cap
        assert gn(FAKE, FAKE, FAKE, FAKE, FAKE, E, m_fit + 1, 256, 256, FAKE, 0, NULL) == 6
    assert "scratch" in fp8bs.status_string(6)


def test_linear_workspace_and_validation(fp8bs):
    """fp8_block_linear: no workspace for the fused decode shapes (at most 16 rows, 8 <= K/128 <= 128,
    N a multiple of 32 with N/32 >= 256); elsewhere the quantized activations (codes, then fp32
    scales, each 16-byte aligned) and the GEMM's own workspace."""
    L = fp8bs.lib()
    wsz = L.fp8bs_linear_workspace_size
    assert wsz(1, 28672, 4096) == 0 and wsz(16, 8192, 1024) == 0 and wsz(5, 16384, 16384) == 0
    assert wsz(0, 128, 128) == 0 and wsz(-1, 128, 1024) == 0

    def a16(b):
        return (b + 15) // 16 * 16
    for M, N, K in ((17, 4096, 4096), (8192, 4096, 4096), (16, 256, 512), (3, 256, 32768), (64, 28672, 4096),
                    (16, 4096, 14336), (1, 8064, 4096), (2, 8192, 896), (1, 8192, 16512)):
        assert wsz(M, N, K) == a16(M * K) + a16(M * (K // 128) * 4) + L.fp8bs_gemm_workspace_size(M, N, K)
    for f in (L.fp8_block_linear, L.fp8_block_linear_pow2):
        assert f(FAKE, FAKE, FAKE, 8, 100, 1024, FAKE, 0, NULL, 0, NULL) == 2     # N % 128
        assert f(FAKE, FAKE, FAKE, 8, 128, 1000, FAKE, 0, NULL, 0, NULL) == 2    # K % 128
        assert f(FAKE, FAKE, FAKE, -1, 128, 1024, FAKE, 0, NULL, 0, NULL) == 1   # M < 0
        assert f(FAKE, FAKE, FAKE, 8, 128, 1024, FAKE, 3, NULL, 0, NULL) == 1    # out dtype
        assert f(NULL, FAKE, FAKE, 8, 128, 1024, FAKE, 0, NULL, 0, NULL) == 1    # null activations
        assert f(MISAL, FAKE, FAKE, 8, 128, 1024, FAKE, 0, NULL, 0, NULL) == 1   # misaligned activations
        assert f(FAKE, FAKE, NULL, 8, 128, 1024, FAKE, 0, NULL, 0, NULL) == 1    # null weight scales
        assert f(FAKE, FAKE, FAKE, 8, 128, 1024, MISAL, 0, NULL, 0, NULL) == 1   # misaligned output
        assert f(NULL, FAKE, FAKE, 0, 128, 1024, NULL, 0, NULL, 0, NULL) == 0    # M == 0: no-op
        need = wsz(17, 4096, 4096)
        assert f(FAKE, FAKE, FAKE, 17, 4096, 4096, FAKE, 0, NULL, 0, NULL) == 4          # no workspace
        assert f(FAKE, FAKE, FAKE, 17, 4096, 4096, FAKE, 0, FAKE, need - 1, NULL) == 4   # too small
        assert f(FAKE, FAKE, FAKE, 17, 4096, 4096, FAKE, 0, MISAL, need, NULL) == 1      # misaligned


def test_unsupported_device_without_gpu(fp8bs):
    """Valid arguments on a host with no HIP device: UNSUPPORTED_DEVICE, nothing launched."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present")
    L = fp8bs.lib()
    assert L.quant_act_1x128(FAKE, 4, 128, FAKE, FAKE, 0, NULL) == 3
    assert L.fp8_block_gemm(FAKE, FAKE, FAKE, FAKE, 8, 128, 128, FAKE, 0, NULL, 0, NULL) == 3
