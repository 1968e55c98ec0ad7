"""GPU parity of the whole linear layer from bf16 activations (fp8_block_linear).

The entry point quantizes X per 1x128 block and multiplies: for one row
(M = 1, K <= 16384) inside the vector-ALU GEMV, for other decode rows
(M <= 16, 8 <= K/128 <= 128, W tiles of 32 or 64 rows) inside the
weight-streaming GEMM, elsewhere through the quantizer and the GEMM.  Gates, on the same seeded bf16 inputs:
- against the oracle's own composition, its quant_act_1x128 then its GEMM:
  max |Y_gpu - Y_oracle| <= 1e-2 * rms(Y_oracle) on the fp32 output;
- bf16 output == round-to-nearest-even of the fp32 output, bit for bit;
- bit for bit the fp32 output of the library's two separate calls
  (quant_act_1x128, then fp8_block_gemm or its _pow2 form), and
  deterministic across calls.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16_to_dev, gemm_gate, host, sample_positions, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.lib()
    return m


FUSED = [
    # one 16-row X tile; W tiles of 64 / 32 rows; K/128 from the smallest (8) to the largest (128)
    (1, 28672, 4096), (16, 28672, 4096), (7, 8192, 1024), (2, 8192, 16384), (12, 16384, 1152), (9, 8192, 3072),
]
UNFUSED = [
    # 16-row W tiles (N/32 < 256), more rows, too few K blocks for the weight-streaming kernel, or too many
    (16, 4096, 14336), (5, 512, 2048), (1, 256, 1024), (17, 4096, 4096), (256, 512, 512), (16, 256, 512),
    (3, 256, 32768), (300, 512, 4096),
    # one row: the GEMV quantizes it in-kernel whatever the workspace query says
    (1, 4096, 14336), (1, 512, 640),
]


def _linear_case(fp8bs, orc, M, N, K, mode, sampled=False):
    x = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_X + 7)
    w = synth.weights(N, K, seed=synth.SEED, sub=synth.SUB_W + 7)
    xd, wd = bf16_to_dev(x), bf16_to_dev(w)
    wq, ws = fp8bs.quant_w_128x128(wd, mode)
    lin = fp8bs.fp8_block_linear_pow2 if mode == 1 else fp8bs.fp8_block_linear
    gem = fp8bs.fp8_block_gemm_pow2 if mode == 1 else fp8bs.fp8_block_gemm
    y32 = lin(xd, wq, ws, out_dtype=torch.float32)
    y16 = lin(xd, wq, ws, out_dtype=torch.bfloat16)
    assert torch.equal(y16.view(torch.int16), y32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(y32.view(torch.int32), lin(xd, wq, ws, out_dtype=torch.float32).view(torch.int32))
    xq, xs = fp8bs.quant_act_1x128(xd, mode)
    ysep = gem(xq, xs, wq, ws, out_dtype=torch.float32)
    assert torch.equal(y32.view(torch.int32), ysep.view(torch.int32)), "differs from the separate calls"
    xq_r, xs_r = orc.quant_act_1x128(x, mode)
    wq_r, ws_r = orc.quant_w_128x128(w, mode)
    if sampled:
        rows, cols = sample_positions(M, N, 3000, seed=M + N + K)
        gemm_gate("Y fp32 (sampled %d)" % rows.size, host(y32)[rows, cols],
                  orc.gemm_sampled(xq_r, xs_r, wq_r, ws_r, rows, cols))
    else:
        gemm_gate("Y fp32", host(y32), orc.gemm(xq_r, xs_r, wq_r, ws_r))


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", FUSED + UNFUSED, ids=lambda s: "%dx%dx%d" % s)
def test_linear_parity(fp8bs, orc, shape, mode):
    M, N, K = shape
    fused = fp8bs.linear_workspace_size(M, N, K) == 0
    say("fp8_block_linear M=%d N=%d K=%d mode=%d fused=%d" % (M, N, K, mode, fused))
    assert fused == (shape in FUSED)
    _linear_case(fp8bs, orc, M, N, K, mode, sampled=M * N * K > (1 << 28))


def test_linear_zero_and_outlier_blocks(fp8bs, orc):
    """All-zero 1x128 blocks (scale 1, codes 0) and a lone huge value per block, fused path."""
    M, N, K = 9, 8192, 2048
    x = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_X + 8)
    x[0, :] = 0                      # a whole zero row
    x[3, 256:384] = 0                # one zero block
    x[5, 130] = np.uint16(0x4780)    # 65536 inside an ordinary block
    x[6, 7] = np.uint16(0xC780)      # -65536
    w = synth.weights(N, K, seed=synth.SEED, sub=synth.SUB_W + 8)
    xd, wd = bf16_to_dev(x), bf16_to_dev(w)
    for mode in (0, 1):
        wq, ws = fp8bs.quant_w_128x128(wd, mode)
        lin = fp8bs.fp8_block_linear_pow2 if mode == 1 else fp8bs.fp8_block_linear
        y32 = lin(xd, wq, ws, out_dtype=torch.float32)
        xq_r, xs_r = orc.quant_act_1x128(x, mode)
        wq_r, ws_r = orc.quant_w_128x128(w, mode)
        ref = orc.gemm(xq_r, xs_r, wq_r, ws_r)
        gemm_gate("Y fp32 mode %d" % mode, host(y32), ref)
        assert np.all(host(y32)[0] == 0.0)


def test_linear_empty(fp8bs):
    x = torch.empty((0, 1024), dtype=torch.bfloat16, device="cuda")
    wq = torch.zeros((128, 1024), dtype=torch.uint8, device="cuda")
    ws = torch.ones((1, 8), dtype=torch.float32, device="cuda")
    assert fp8bs.fp8_block_linear(x, wq, ws).shape == (0, 128)
