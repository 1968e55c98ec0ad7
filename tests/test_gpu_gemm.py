"""GPU parity of the block-scaled GEMM and the grouped (MoE) GEMM.

End to end on the same seeded bf16 inputs: the GPU path quantizes and
multiplies with the library; the oracle quantizes and multiplies with its own
code.  Gate (fp32 output mode): max |Y_gpu - Y_oracle| <= 1e-2 * rms(Y_oracle).
The bf16 output must equal the round-to-nearest-even of the fp32 output bit
for bit.  Shapes: the tiny layer, ragged shapes that leave partial tiles, the
8B-shaped dense layers, the decode grid and the MoE layer at full size
(every output, against the oracle's full-output GEMMs).
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitexact, bf16_to_dev, gemm_gate, host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.lib()
    return m


def _pow2_outputs(fn, *args):
    """fp32 and bf16 outputs of a _pow2 entry point (the matrix cores apply the scales)."""
    y32 = fn(*args, out_dtype=torch.float32)
    y16 = fn(*args, out_dtype=torch.bfloat16)
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    y32b = fn(*args, out_dtype=torch.float32)
    assert torch.equal(y32.view(torch.int32), y32b.view(torch.int32))
    return y32


def _run_pair(fp8bs, orc, M, N, K, mode, seed_sub=0):
    x = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_X + 10 * seed_sub)
    w = synth.weights(N, K, seed=synth.SEED, sub=synth.SUB_W + 10 * seed_sub)
    xd, wd = bf16_to_dev(x), bf16_to_dev(w)
    xq, xs = fp8bs.quant_act_1x128(xd, mode)
    wq, ws = fp8bs.quant_w_128x128(wd, mode)
    y32 = fp8bs.fp8_block_gemm(xq, xs, wq, ws, out_dtype=torch.float32)
    y16 = fp8bs.fp8_block_gemm(xq, xs, wq, ws, out_dtype=torch.bfloat16)
    ref_q = orc.quant_act_1x128(x, mode), orc.quant_w_128x128(w, mode)
    return (x, w, xd, wd, xq, xs, wq, ws, y32, y16, ref_q)


SMALL = [
    (256, 512, 512),    # tiny layer
    (1, 128, 128), (17, 256, 384), (129, 384, 640), (300, 128, 1024), (127, 640, 256), (513, 1024, 1152),
    # few-row shapes of the weight-streaming path: 1 / 2 / 4 / 8 sixteen-row X tiles (ragged M, two
    # X-row chunks at M = 256), 16 / 32 / 64-row W tiles, K blocks not a multiple of the 8 waves
    (1, 256, 1024), (5, 512, 2048), (16, 1024, 1152), (24, 16384, 1024), (33, 512, 1024), (64, 2048, 1280),
    (100, 384, 2048), (256, 128, 1024), (7, 8192, 1024),
    # 64-row persistent tiles up to 128 rows: ragged second row tile, and two full ones split along K
    (100, 768, 2048), (128, 1024, 4096),
    # products split along K (fewer output tiles than compute units): 16 ranges of 4 blocks, uneven
    # ranges of 4 and 5 blocks (K/128 = 23), and 256-row tiles with a ragged second row tile
    (40, 512, 8192), (97, 512, 2944), (300, 512, 4096),
    # a few rows with K past the weight-streaming kernel's 16384: the persistent kernel, 32 K ranges
    (3, 256, 32768),
    # one activation row (the vector-ALU GEMV): all 16 K chunks, a partial last chunk, past its K limit
    (1, 512, 16384), (1, 384, 640), (1, 256, 16512),
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "%dx%dx%d" % s)
def test_gemm_parity_full_output(fp8bs, orc, shape, mode):
    M, N, K = shape
    say("fp8_block_gemm M=%d N=%d K=%d mode=%d" % (M, N, K, mode))
    x, w, xd, wd, xq, xs, wq, ws, y32, y16, ((xq_r, xs_r), (wq_r, ws_r)) = _run_pair(fp8bs, orc, M, N, K, mode)
    assert_bitexact("xq", host(xq), xq_r)
    assert_bitexact("wq", host(wq), wq_r)
    ref = orc.gemm(xq_r, xs_r, wq_r, ws_r)
    gemm_gate("Y fp32", host(y32), ref)
    # bf16 output == RNE_bf16(fp32 output), bit for bit
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    # deterministic: a second run is bit-identical
    y32b = fp8bs.fp8_block_gemm(xq, xs, wq, ws, out_dtype=torch.float32)
    assert torch.equal(y32.view(torch.int32), y32b.view(torch.int32))
    if mode == 1:
        # power-of-2 scales: the entry point that hands them to the matrix cores
        gemm_gate("Y fp32 (pow2 entry)", host(_pow2_outputs(fp8bs.fp8_block_gemm_pow2, xq, xs, wq, ws)), ref)
    # reported, not gated: error against the unquantized bf16 product
    yb = (xd.float() @ wd.float().T)
    say("  vs unquantized bf16 GEMM: max|err|/rms = %.3e" %
        float((y32 - yb).abs().max() / yb.pow(2).mean().sqrt()))


# The 256x256 persistent kernel with units of one to three K blocks: every step, or every other one,
# ends a tile while the next tile's first W fragments are already being read (three MFMA groups
# ahead); a ragged last row tile (M = 4000) and 17 column tiles (N = 4352).  Every output is checked.
SHORT_K_256 = [(4096, 4096, 128), (4000, 4096, 384), (4096, 4352, 256)]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", SHORT_K_256, ids=lambda s: "%dx%dx%d" % s)
def test_gemm_256x256_short_k_full_output(fp8bs, orc, shape, mode):
    M, N, K = shape
    say("fp8_block_gemm (256x256 tiles, short K) M=%d N=%d K=%d mode=%d" % (M, N, K, mode))
    x, w, xd, wd, xq, xs, wq, ws, y32, y16, ((xq_r, xs_r), (wq_r, ws_r)) = _run_pair(fp8bs, orc, M, N, K, mode)
    assert_bitexact("xq", host(xq), xq_r)
    assert_bitexact("wq", host(wq), wq_r)
    ref = orc.gemm_full(xq_r, xs_r, wq_r, ws_r)
    gemm_gate("Y fp32", host(y32), ref)
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    if mode == 1:
        gemm_gate("Y fp32 (pow2 entry)", host(_pow2_outputs(fp8bs.fp8_block_gemm_pow2, xq, xs, wq, ws)), ref)


def test_gemm_integer_special_case(fp8bs):
    """Codes of small integers with unit scales: the product is an exact integer
    matmul, which fp32 accumulation reproduces exactly at this size."""
    g = np.random.default_rng(5)
    codes = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], dtype=np.uint8)
    M, N, K = 200, 256, 512
    ix, iw = g.integers(0, 9, (M, K)), g.integers(0, 9, (N, K))
    sx, sw = g.integers(0, 2, (M, K)), g.integers(0, 2, (N, K))
    xq = codes[ix] | (sx * 0x80).astype(np.uint8)
    wq = codes[iw] | (sw * 0x80).astype(np.uint8)
    ref = ((ix * (1 - 2 * sx)) @ (iw * (1 - 2 * sw)).T).astype(np.float32)
    y = fp8bs.fp8_block_gemm(to_dev(xq), to_dev(np.ones((M, K // 128), np.float32)), to_dev(wq),
                             to_dev(np.ones((N // 128, K // 128), np.float32)), out_dtype=torch.float32)
    assert np.array_equal(host(y), ref)
    # unit scales are powers of two: the scaled-MFMA path is exact here too, and so are other
    # power-of-2 scales (2^-3 on X, 2^5 on W multiply the exact integer result by 4)
    y = fp8bs.fp8_block_gemm_pow2(to_dev(xq), to_dev(np.ones((M, K // 128), np.float32)), to_dev(wq),
                                  to_dev(np.ones((N // 128, K // 128), np.float32)), out_dtype=torch.float32)
    assert np.array_equal(host(y), ref)
    y = fp8bs.fp8_block_gemm_pow2(to_dev(xq), to_dev(np.full((M, K // 128), 0.125, np.float32)), to_dev(wq),
                                  to_dev(np.full((N // 128, K // 128), 32.0, np.float32)), out_dtype=torch.float32)
    assert np.array_equal(host(y), 4 * ref)


@pytest.mark.parametrize("shape", [(300, 512, 1024), (4096, 4096, 256)], ids=["split_128x256", "256x256"])
def test_gemm_pow2_scale_products_below_normal_range(fp8bs, orc, shape):
    """Power-of-2 scales whose products fall below fp32's normal range (2^-64 * 2^-64 = 2^-128), or
    mix tiny and large factors, down to the smallest E8M0 scale 2^-127: each factor rides its own
    operand's E8M0 scale, so the POW2 entry point matches the oracle (a single E8M0 code for the
    product read 2^-128 as 2^-127, off by a factor of 2)."""
    M, N, K = shape
    g = np.random.default_rng(M + K)
    xq = g.integers(0, 256, (M, K), dtype=np.uint8)
    wq = g.integers(0, 256, (N, K), dtype=np.uint8)
    xq[(xq & 0x7F) == 0x7F] = 0x3F
    wq[(wq & 0x7F) == 0x7F] = 0x3F
    for ex, ew in ((-64, -64), (-100, 60), (-127, 20), (40, -127), (-70, -50)):
        jx = g.integers(-2, 3, (M, K // 128))
        jw = g.integers(-2, 3, (N // 128, K // 128))
        xs = np.ldexp(1.0, np.maximum(ex + jx, -127)).astype(np.float32)
        ws = np.ldexp(1.0, np.maximum(ew + jw, -127)).astype(np.float32)
        say("fp8_block_gemm_pow2 M=%d N=%d K=%d scale exponents around %d, %d" % (M, N, K, ex, ew))
        y = fp8bs.fp8_block_gemm_pow2(to_dev(xq), to_dev(xs), to_dev(wq), to_dev(ws), out_dtype=torch.float32)
        gemm_gate("Y fp32 (pow2 entry)", host(y), orc.gemm_full(xq, xs, wq, ws))


def test_gemm_empty(fp8bs):
    xq = torch.empty((0, 256), dtype=torch.uint8, device="cuda")
    xs = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    wq = torch.zeros((128, 256), dtype=torch.uint8, device="cuda")
    ws = torch.ones((1, 2), dtype=torch.float32, device="cuda")
    y = fp8bs.fp8_block_gemm(xq, xs, wq, ws)
    assert y.shape == (0, 128)


# 8B-shaped dense layers (M = 8192) and the decode grid (M in {1, 16, 64, 128, 256} against the
# gate+up and down weights), full size, every output
LARGE = [
    ("qkv", 8192, 6144, 4096), ("gate_up", 8192, 28672, 4096), ("down", 8192, 4096, 14336),
    ("o_proj", 8192, 4096, 4096),
] + [("decode%d_%s" % (m, name), m, n, k) for m in (1, 16, 64, 128, 256)
     for name, n, k in (("gate_up", 28672, 4096), ("down", 4096, 14336))] + [
    # one K block per tile and more tiles than workgroups: every workgroup walks several one-step tiles
    ("k128_many_tiles", 4352, 4096, 128),
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("case", LARGE, ids=lambda c: c[0])
def test_gemm_parity_full_size(fp8bs, orc, case, mode):
    name, M, N, K = case
    say("fp8_block_gemm %s M=%d N=%d K=%d mode=%d" % (name, M, N, K, mode))
    x, w, xd, wd, xq, xs, wq, ws, y32, y16, ((xq_r, xs_r), (wq_r, ws_r)) = _run_pair(fp8bs, orc, M, N, K, mode)
    assert_bitexact("xq", host(xq), xq_r)
    assert_bitexact("xs", host(xs), xs_r)
    assert_bitexact("wq", host(wq), wq_r)
    assert_bitexact("ws", host(ws), ws_r)
    del x, w, xd, wd
    ref = orc.gemm_full(xq_r, xs_r, wq_r, ws_r)
    gemm_gate("Y fp32 (all %d outputs)" % ref.size, host(y32), ref)
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    del y16
    if mode == 1:
        del y32
        gemm_gate("Y fp32 (pow2 entry, all %d outputs)" % ref.size,
                  host(_pow2_outputs(fp8bs.fp8_block_gemm_pow2, xq, xs, wq, ws)), ref)


# ---- grouped (MoE) ---------------------------------------------------------------

def _grouped(fp8bs, orc, counts, N, K, mode, token_rows=None, x_tok=None, seed_sub=0):
    offs = synth.offsets_from_counts(counts)
    M = int(offs[-1])
    E = len(counts)
    if x_tok is not None:
        x = np.ascontiguousarray(x_tok[token_rows])
    else:
        x = synth.activations(max(M, 1), K, seed=synth.SEED, sub=synth.SUB_X + seed_sub)[:M]
    w = synth.expert_weights(E, N, K, seed=synth.SEED, sub=synth.SUB_W + seed_sub)
    xq, xs = fp8bs.quant_act_1x128(bf16_to_dev(x), mode)
    wd = bf16_to_dev(w.reshape(E * N, K))
    wq, ws = fp8bs.quant_w_128x128(wd, mode)  # experts stacked along N: the same 128x128 blocks
    wq = wq.view(E, N, K)
    ws = ws.view(E, N // 128, K // 128)
    offs_d = to_dev(offs)
    y32 = fp8bs.fp8_block_grouped_gemm(xq, xs, wq, ws, offs_d, out_dtype=torch.float32)
    y16 = fp8bs.fp8_block_grouped_gemm(xq, xs, wq, ws, offs_d, out_dtype=torch.bfloat16)
    if mode == 1:  # power-of-2 scales: the scaled-MFMA entry point, gated by the callers like y32
        y32 = (y32, _pow2_outputs(fp8bs.fp8_block_grouped_gemm_pow2, xq, xs, wq, ws, offs_d))
    xq_r, xs_r = orc.quant_act_1x128(x, mode)
    wq_r, ws_r = orc.quant_w_128x128(w.reshape(E * N, K), mode)
    wq_r = wq_r.reshape(E, N, K)
    ws_r = ws_r.reshape(E, N // 128, K // 128)
    assert_bitexact("xq", host(xq), xq_r)
    assert_bitexact("wq", host(wq), wq_r)
    return xq_r, xs_r, wq_r, ws_r, offs, y32, y16


GROUP_COUNTS = [
    [5, 0, 129, 1, 64, 300],     # empty, one-row and ragged experts
    [0, 0, 0, 7],
    [128, 128, 256],
    [1] * 70,                     # more experts than one wave's lanes
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("counts", GROUP_COUNTS, ids=["ragged", "leading_empty", "aligned", "e70"])
def test_grouped_parity(fp8bs, orc, counts, mode):
    N, K = 256, 384
    say("fp8_block_grouped_gemm counts=%s mode=%d" % (counts[:8], mode))
    xq_r, xs_r, wq_r, ws_r, offs, y32, y16 = _grouped(fp8bs, orc, counts, N, K, mode, seed_sub=len(counts))
    ref = orc.grouped_gemm(xq_r, xs_r, wq_r, ws_r, offs)
    if mode == 1:
        y32, yp = y32
        gemm_gate("Y fp32 (pow2 entry)", host(yp), ref)
    gemm_gate("Y fp32", host(y32), ref)
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_grouped_parity_moe_full_size(fp8bs, orc, proj, mode):
    """128 experts, hidden 2048, expert FFN 768, 8192 tokens routed top-8; every output."""
    row_token, offs = synth.moe_routing(8192, 128, 8)
    counts = np.diff(offs)
    if proj == "gate_up":
        N, K = 1536, 2048
        x_tok = synth.activations(8192, K, seed=synth.SEED, sub=synth.SUB_X)
        args = dict(token_rows=row_token, x_tok=x_tok)
    else:
        N, K = 2048, 768
        args = {}
    say("fp8_block_grouped_gemm MoE %s M=%d N=%d K=%d mode=%d" % (proj, offs[-1], N, K, mode))
    xq_r, xs_r, wq_r, ws_r, offs, y32, y16 = _grouped(fp8bs, orc, counts, N, K, mode, **args)
    ref = orc.grouped_gemm_full(xq_r, xs_r, wq_r, ws_r, offs)
    if mode == 1:
        y32, yp = y32
        gemm_gate("Y fp32 (pow2 entry, all %d outputs)" % ref.size, host(yp), ref)
    gemm_gate("Y fp32 (all %d outputs)" % ref.size, host(y32), ref)
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
