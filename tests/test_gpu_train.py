"""GPU parity of the training path's weight quantizer and data-gradient product.

quant_w_128x128_dual writes the codes and scales of W and of W^T from one read
of W.  Bar: bit-exact against the oracle -- (wq, ws) against its quantization
of W, (wqt, wst) against its quantization of the transposed matrix (small
shapes) or, at full size, against the transpose of its quantization of W
(the oracle's transpose symmetry is pinned on the CPU).  The data gradient
dX = dY W runs fp8_block_gemm on quant_act_1x128(dY) and (wqt, wst); its gate
is the GEMM gate against the oracle's fp64 product of the same quantized
operands.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitexact, bf16_to_dev, gemm_gate, host, sample_positions, say

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
def test_dgrad_parity_full_size_sampled(fp8bs, orc, case):
    name, N, K = case
    M = 8192
    say("dgrad %s M=%d N=%d K=%d" % (name, M, N, K))
    dx32, dyq_r, dys_r, wqt_r, wst_r = _dgrad(fp8bs, orc, M, N, K, 0)
    rows, cols = sample_positions(M, K, 3000, seed=M + N + K)
    ref = orc.gemm_sampled(dyq_r, dys_r, wqt_r, wst_r, rows, cols)
    gemm_gate("dX fp32 (sampled %d)" % rows.size, host(dx32)[rows, cols], ref)
