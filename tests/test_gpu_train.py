"""GPU parity of the training path: the data and weight gradients' quantizers and products.

quant_w_128x128_dual writes the codes and scales of W and of W^T from one read
of W.  Bar: bit-exact against the oracle -- (wq, ws) against its quantization
of W, (wqt, wst) against its quantization of the transposed matrix (small
shapes) or, at full size, against the transpose of its quantization of W
(the oracle's transpose symmetry is pinned on the CPU).  The data gradient
dX = dY W runs fp8_block_gemm on quant_act_1x128(dY) and (wqt, wst); its gate
is the GEMM gate against the oracle's fp64 product of the same quantized
operands.  The weight gradient dW = dY^T X quantizes both operands with
quant_act_1x128_t (bit-exact against the oracle's quant_act_1x128 of the
transposed matrix) and multiplies them with fp8_block_gemm_1x128.  Both of
its operands carry the x50 outliers, whose coinciding products make some
outputs ~100x the rms; there the matrix core's own dot-product precision
(below 2^-12 of a block's sum of |products|, pinned here) exceeds 1e-2 * rms,
so its gate adds the standard dot-product term tau * sum |products|
(tau = 2^-11) to the 1e-2 * rms of the forward GEMM gate.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import (MFMA_DOT_TAU, assert_bitexact, bf16_to_dev, gemm_gate, gemm_gate_abs, host, sample_positions,
                      say, to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.lib()
    return m


SMALL_W = [(128, 128), (512, 512), (384, 256), (256, 1152), (1536, 2048), (2048, 768)]
FULL_W = [(6144, 4096), (28672, 4096), (4096, 14336), (4096, 4096)]


def _check_dual(orc, w, outs, mode, direct_transpose):
    wq, ws, wqt, wst = (host(t) for t in outs)
    q_ref, s_ref = orc.quant_w_128x128(w, mode)
    assert_bitexact("wq", wq, q_ref)
    assert_bitexact("ws", ws, s_ref)
    if direct_transpose:
        qt_ref, st_ref = orc.quant_w_128x128(np.ascontiguousarray(w.T), mode)
    else:
        qt_ref, st_ref = np.ascontiguousarray(q_ref.T), np.ascontiguousarray(s_ref.T)
    assert_bitexact("wqt", wqt, qt_ref)
    assert_bitexact("wst", wst, st_ref)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", SMALL_W + FULL_W, ids=lambda s: "%dx%d" % s)
def test_quant_w_dual_parity(fp8bs, orc, shape, mode):
    N, K = shape
    say("quant_w_128x128_dual N=%d K=%d mode=%d" % (N, K, mode))
    w = synth.weights(N, K, seed=synth.SEED, sub=synth.sub_layer(0))
    outs = fp8bs.quant_w_128x128_dual(bf16_to_dev(w), mode)
    _check_dual(orc, w, outs, mode, direct_transpose=shape in SMALL_W)


@pytest.mark.parametrize("mode", [0, 1])
def test_quant_w_dual_batched_parity(fp8bs, orc, mode):
    """40 tensors of mixed shapes in one call (more than one launch's worth)."""
    shapes = [(128 * (1 + (i * 3) % 7), 128 * (1 + (i * 5) % 6)) for i in range(40)]
    say("quant_w_128x128_dual_batched %d tensors mode=%d" % (len(shapes), mode))
    ws = [synth.weights(n, k, seed=synth.SEED, sub=synth.sub_layer(i)) for i, (n, k) in enumerate(shapes)]
    outs = fp8bs.quant_w_128x128_dual_batched([bf16_to_dev(w) for w in ws], mode)
    for i, (w, o) in enumerate(zip(ws, outs)):
        _check_dual(orc, w, o, mode, direct_transpose=True)


def test_quant_w_dual_special_blocks(fp8bs, orc):
    """Zero, signed-zero and extreme blocks keep their codes through the transpose."""
    N, K = 256, 384
    w = synth.weights(N, K, seed=synth.SEED, sub=synth.sub_layer(7)).copy()
    w[0:128, 0:128] = 0                      # all +0
    w[0:128, 128:256] = 0x8000               # all -0
    w[128:256, 0:128] = 0x7F7F               # the largest finite bf16
    w[128:256, 0:128:2] |= 0x8000
    w[128:256, 256:384] = np.arange(128 * 128, dtype=np.uint16).reshape(128, 128) % 0x80 + 1  # subnormals
    for mode in (0, 1):
        outs = fp8bs.quant_w_128x128_dual(bf16_to_dev(w), mode)
        _check_dual(orc, w, outs, mode, direct_transpose=True)


def _dgrad(fp8bs, orc, M, N, K, mode):
    """dX [M, K] = dY [M, N] W [N, K]: (dYq, dYs) along N times (Wq^T, Ws^T)."""
    dy = synth.activations(M, N, seed=synth.SEED, sub=synth.SUB_DY)
    w = synth.weights(N, K, seed=synth.SEED, sub=synth.SUB_W)
    dyq, dys = fp8bs.quant_act_1x128(bf16_to_dev(dy), mode)
    _, _, wqt, wst = fp8bs.quant_w_128x128_dual(bf16_to_dev(w), mode)
    dx32 = fp8bs.fp8_block_gemm(dyq, dys, wqt, wst, out_dtype=torch.float32)
    dx16 = fp8bs.fp8_block_gemm(dyq, dys, wqt, wst, out_dtype=torch.bfloat16)
    assert torch.equal(dx16.view(torch.int16), dx32.to(torch.bfloat16).view(torch.int16))
    dyq_r, dys_r = orc.quant_act_1x128(dy, mode)
    wq_r, ws_r = orc.quant_w_128x128(w, mode)
    assert_bitexact("dyq", host(dyq), dyq_r)
    assert_bitexact("dys", host(dys), dys_r)
    return dx32, dyq_r, dys_r, np.ascontiguousarray(wq_r.T), np.ascontiguousarray(ws_r.T)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", [(256, 512, 512), (130, 1152, 640), (513, 384, 1024), (16, 2048, 768)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_dgrad_parity_full_output(fp8bs, orc, shape, mode):
    M, N, K = shape
    say("dgrad M=%d N=%d K=%d mode=%d" % (M, N, K, mode))
    dx32, dyq_r, dys_r, wqt_r, wst_r = _dgrad(fp8bs, orc, M, N, K, mode)
    gemm_gate("dX fp32", host(dx32), orc.gemm(dyq_r, dys_r, wqt_r, wst_r))


# the data gradients of the 8B-shaped dense layers at M = 8192 tokens: (N, K) of the forward weight
DGRAD_LARGE = [("qkv", 6144, 4096), ("gate_up", 28672, 4096), ("down", 4096, 14336), ("o_proj", 4096, 4096)]


@pytest.mark.parametrize("case", DGRAD_LARGE, ids=lambda c: c[0])
def test_dgrad_parity_full_size(fp8bs, orc, case):
    name, N, K = case
    M = 8192
    say("dgrad %s M=%d N=%d K=%d" % (name, M, N, K))
    dx32, dyq_r, dys_r, wqt_r, wst_r = _dgrad(fp8bs, orc, M, N, K, 0)
    ref = orc.gemm_full(dyq_r, dys_r, wqt_r, wst_r)
    gemm_gate("dX fp32 (all %d outputs)" % ref.size, host(dx32), ref)


# ---- weight gradient: dW = dY^T X, both operands in 1x128 blocks along the tokens ----

ACT_T_SHAPES = [(128, 128), (256, 512), (384, 1152), (1024, 768), (8192, 4096), (8192, 28672)]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", ACT_T_SHAPES, ids=lambda s: "%dx%d" % s)
def test_quant_act_t_parity(fp8bs, orc, shape, mode):
    M, K = shape
    say("quant_act_1x128_t M=%d K=%d mode=%d" % (M, K, mode))
    x = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_X)
    q_ref, s_ref = orc.quant_act_1x128_t(x, mode)
    q, s = fp8bs.quant_act_1x128_t(bf16_to_dev(x), mode)
    assert_bitexact("codes", host(q), q_ref)
    assert_bitexact("scales", host(s), s_ref)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", [(128, 128), (384, 1152), (8192, 4096), (8192, 28672)], ids=lambda s: "%dx%d" % s)
def test_quant_act_dual_parity(fp8bs, orc, shape, mode):
    """Both quantizations of an output gradient from one read: bit-exact against the
    oracle's quant_act_1x128 of dY and of dY^T."""
    M, K = shape
    say("quant_act_1x128_dual M=%d K=%d mode=%d" % (M, K, mode))
    dy = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_DY)
    xq, xs, xqt, xst = fp8bs.quant_act_1x128_dual(bf16_to_dev(dy), mode)
    q_ref, s_ref = orc.quant_act_1x128(dy, mode)
    assert_bitexact("row codes", host(xq), q_ref)
    assert_bitexact("row scales", host(xs), s_ref)
    qt_ref, st_ref = orc.quant_act_1x128_t(dy, mode)
    assert_bitexact("transposed codes", host(xqt), qt_ref)
    assert_bitexact("transposed scales", host(xst), st_ref)


def _wgrad(fp8bs, orc, M, N, K, mode):
    """dW [N, K] = dY [M, N]^T X [M, K] over M tokens."""
    dy = synth.activations(M, N, seed=synth.SEED, sub=synth.SUB_DY)
    x = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_X)
    dyq, dys = fp8bs.quant_act_1x128_t(bf16_to_dev(dy), mode)
    xq, xs = fp8bs.quant_act_1x128_t(bf16_to_dev(x), mode)
    dw32 = fp8bs.fp8_block_gemm_1x128(dyq, dys, xq, xs, out_dtype=torch.float32)
    dw16 = fp8bs.fp8_block_gemm_1x128(dyq, dys, xq, xs, out_dtype=torch.bfloat16)
    assert torch.equal(dw16.view(torch.int16), dw32.to(torch.bfloat16).view(torch.int16))
    dw32b = fp8bs.fp8_block_gemm_1x128(dyq, dys, xq, xs, out_dtype=torch.float32)
    assert torch.equal(dw32.view(torch.int32), dw32b.view(torch.int32))
    outs = [("dW fp32", dw32)]
    if mode == 1:  # power-of-2 scales: the entry point that hands both scales to the matrix cores
        p32 = fp8bs.fp8_block_gemm_1x128_pow2(dyq, dys, xq, xs, out_dtype=torch.float32)
        p16 = fp8bs.fp8_block_gemm_1x128_pow2(dyq, dys, xq, xs, out_dtype=torch.bfloat16)
        assert torch.equal(p16.view(torch.int16), p32.to(torch.bfloat16).view(torch.int16))
        p32b = fp8bs.fp8_block_gemm_1x128_pow2(dyq, dys, xq, xs, out_dtype=torch.float32)
        assert torch.equal(p32.view(torch.int32), p32b.view(torch.int32))
        outs.append(("dW fp32 (pow2 entry)", p32))
    dyq_r, dys_r = orc.quant_act_1x128_t(dy, mode)
    xq_r, xs_r = orc.quant_act_1x128_t(x, mode)
    assert_bitexact("dyq", host(dyq), dyq_r)
    assert_bitexact("xq", host(xq), xq_r)
    return outs, dyq_r, dys_r, xq_r, xs_r


def test_mfma_dot_product_precision(fp8bs, orc):
    """Pins the relative factor of the weight-gradient gate: one dominant product
    (448 x 448) beside 127 small ones, and one K block of the outlier data, each
    within MFMA_DOT_TAU of their sum of |products| on the matrix cores."""
    dec = orc.e4m3_decode_array
    cases = []
    for small in (0x38, 0x30, 0x28, 0x20, 0x10, 0x08, 0x01):
        a = np.full(128, small, np.uint8)
        b = np.full(128, 0x38, np.uint8)
        a[0] = b[0] = 0x7E
        cases.append((a, b))
    g = np.random.default_rng(3)
    for _ in range(8):        # random codes of both signs, one +-448 x +-448 product each
        a = g.integers(0, 0x7E, 128).astype(np.uint8) | (g.integers(0, 2, 128) << 7).astype(np.uint8)
        b = g.integers(0, 0x7E, 128).astype(np.uint8) | (g.integers(0, 2, 128) << 7).astype(np.uint8)
        a[5], b[5] = 0x7E, 0xFE
        cases.append((a, b))
    worst = 0.0
    for a, b in cases:
        A = np.zeros((1, 128), np.uint8)
        B = np.zeros((128, 128), np.uint8)
        A[0], B[0] = a, b
        y = host(fp8bs.fp8_block_gemm_1x128(to_dev(A), to_dev(np.ones((1, 1), np.float32)), to_dev(B),
                                            to_dev(np.ones((128, 1), np.float32)), out_dtype=torch.float32))[0, 0]
        prods = dec(a).astype(np.float64) * dec(b).astype(np.float64)
        rel = abs(float(y) - prods.sum()) / np.abs(prods).sum()
        worst = max(worst, rel)
    say("FP8 MFMA dot product: worst |P_gpu - P| / sum|products| = %.3e (2^%.1f)" % (worst, np.log2(max(worst, 1e-30))))
    assert worst <= MFMA_DOT_TAU


def _abs_codes(q):
    return q & np.uint8(0x7F)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", [
    (256, 256, 384), (384, 512, 128), (640, 1152, 384),       # input width not a multiple of 256: 128x128 kernel
    (128, 128, 256), (256, 384, 512), (384, 1152, 768),       # the persistent kernel, 128x256 tiles
], ids=lambda s: "%dx%dx%d" % s)
def test_wgrad_parity_full_output(fp8bs, orc, shape, mode):
    M, N, K = shape
    say("wgrad tokens=%d N=%d K=%d mode=%d" % (M, N, K, mode))
    outs, dyq_r, dys_r, xq_r, xs_r = _wgrad(fp8bs, orc, M, N, K, mode)
    ref = orc.gemm_1x128(dyq_r, dys_r, xq_r, xs_r)
    abs_sum = orc.gemm_1x128(_abs_codes(dyq_r), dys_r, _abs_codes(xq_r), xs_r)
    for name, dw32 in outs:
        gemm_gate_abs(name, host(dw32), ref, abs_sum)


# the weight gradients of the 8B-shaped layers over 8192 tokens (persistent kernel, 256x256 tiles), and
# one K step per tile with two tiles per workgroup (the W-row scale slots wrap across tile changes)
WGRAD_LARGE = [(n, N, K, 8192) for n, N, K in DGRAD_LARGE] + [("tokens128_many_tiles", 8192, 4096, 128)]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("case", WGRAD_LARGE, ids=lambda c: c[0])
def test_wgrad_parity_full_size_sampled(fp8bs, orc, case, mode):
    name, N, K, M = case
    say("wgrad %s tokens=%d N=%d K=%d mode=%d" % (name, M, N, K, mode))
    outs, dyq_r, dys_r, xq_r, xs_r = _wgrad(fp8bs, orc, M, N, K, mode)
    rows, cols = sample_positions(N, K, 3000, seed=M + N + K)
    ref = orc.gemm_1x128_sampled(dyq_r, dys_r, xq_r, xs_r, rows, cols)
    abs_sum = orc.gemm_1x128_sampled(_abs_codes(dyq_r), dys_r, _abs_codes(xq_r), xs_r, rows, cols)
    for label, dw32 in outs:
        gemm_gate_abs("%s (sampled %d)" % (label, rows.size), host(dw32)[rows, cols], ref, abs_sum)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", [(200, 256, 384), (77, 512, 1024), (1000, 384, 256), (300, 8192, 512)],
                         ids=lambda s: "%dx%dx%d" % s)
def test_gemm_1x128_ragged_rows(fp8bs, orc, shape, mode):
    """fp8_block_gemm_1x128 (and with power-of-2 scales its _pow2 form) straight from two
    1x128-quantized operands, with row counts that leave partial tiles (the persistent kernel
    where the width is a multiple of 256, the 128x128 kernel elsewhere); both operands carry the
    outlier recipe."""
    M, N, K = shape
    say("fp8_block_gemm_1x128 M=%d N=%d K=%d mode=%d" % (M, N, K, mode))
    a = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_DY)
    b = synth.activations(N, K, seed=synth.SEED, sub=synth.SUB_X)
    aq, as_ = fp8bs.quant_act_1x128(bf16_to_dev(a), mode)
    bq, bs = fp8bs.quant_act_1x128(bf16_to_dev(b), mode)
    fns = [("Y fp32", fp8bs.fp8_block_gemm_1x128)] + ([("Y fp32 (pow2 entry)", fp8bs.fp8_block_gemm_1x128_pow2)]
                                                      if mode else [])
    aq_r, as_r = orc.quant_act_1x128(a, mode)
    bq_r, bs_r = orc.quant_act_1x128(b, mode)
    ref = orc.gemm_1x128(aq_r, as_r, bq_r, bs_r)
    abs_sum = orc.gemm_1x128(_abs_codes(aq_r), as_r, _abs_codes(bq_r), bs_r)
    for label, fn in fns:
        y32 = fn(aq, as_, bq, bs, out_dtype=torch.float32)
        y16 = fn(aq, as_, bq, bs, out_dtype=torch.bfloat16)
        assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
        gemm_gate_abs(label, host(y32), ref, abs_sum)
