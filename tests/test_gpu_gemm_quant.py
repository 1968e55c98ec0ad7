"""GPU parity of fp8_block_gemm_quant: the GEMM whose epilogue also writes the
next layer's 1x128 FP8 input.

For each shape and scale mode:
- its bf16 Y equals fp8_block_gemm's (same kernel main loop), bit for bit;
- its codes and scales equal quant_act_1x128 of that bf16 Y, bit for bit (the
  library's activation quantizer is itself bit-exact against the oracle on
  every (x, amax) pair);
- the same codes and scales come out when Y is not requested;
- against the oracle: the fp32 product passes the GEMM gate, and the
  dequantized output codes lie within the E4M3 rounding bound of the oracle's Y.
Shapes: 8B-shaped layers (fused into the 256x256 kernel's epilogue), a fused
shape with a partial last row tile, and small shapes that take the
GEMM-then-quantizer route.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitexact, bf16_to_dev, gemm_gate, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.lib()
    return m


SHAPES = [
    ("o_proj", 8192, 4096, 4096), ("qkv", 8192, 6144, 4096),
    ("ragged_fused", 8200, 8192, 1024),        # 33 x 32 tiles of 256x256, last row tile 8 rows
    ("small", 300, 512, 1024), ("tiny", 256, 512, 512), ("one_row", 1, 256, 2048),
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("case", SHAPES, ids=lambda c: c[0])
def test_gemm_quant_parity(fp8bs, orc, case, mode):
    name, M, N, K = case
    fused = fp8bs.gemm_quant_workspace_size(M, N, K) == 0
    say("fp8_block_gemm_quant %s M=%d N=%d K=%d mode=%d fused=%d" % (name, M, N, K, mode, fused))
    assert fused == (name in ("o_proj", "qkv", "ragged_fused"))
    x = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_X + 3)
    w = synth.weights(N, K, seed=synth.SEED, sub=synth.SUB_W + 3)
    xq, xs = fp8bs.quant_act_1x128(bf16_to_dev(x), mode)
    wq, ws = fp8bs.quant_w_128x128(bf16_to_dev(w), mode)
    gemm = fp8bs.fp8_block_gemm_pow2 if mode else fp8bs.fp8_block_gemm
    y, yq, ys = fp8bs.fp8_block_gemm_quant(xq, xs, wq, ws, mode)
    y_ref16 = gemm(xq, xs, wq, ws, out_dtype=torch.bfloat16)
    assert torch.equal(y.view(torch.int16), y_ref16.view(torch.int16)), "bf16 Y differs from fp8_block_gemm"
    cq, cs = fp8bs.quant_act_1x128(y, mode)
    assert_bitexact("yq vs quant_act_1x128(Y)", host(yq), host(cq))
    assert_bitexact("ys vs quant_act_1x128(Y)", host(ys), host(cs))
    _, yq2, ys2 = fp8bs.fp8_block_gemm_quant(xq, xs, wq, ws, mode, want_y=False)
    assert torch.equal(yq2, yq) and torch.equal(ys2.view(torch.int32), ys.view(torch.int32))
    # against the oracle
    xq_r, xs_r = orc.quant_act_1x128(x, mode)
    wq_r, ws_r = orc.quant_w_128x128(w, mode)
    assert_bitexact("xq", host(xq), xq_r)
    assert_bitexact("wq", host(wq), wq_r)
    ref = orc.gemm_full(xq_r, xs_r, wq_r, ws_r)
    y32 = gemm(xq, xs, wq, ws, out_dtype=torch.float32)
    gemm_gate("Y fp32", host(y32), ref)
    # dequantized output codes against the oracle's Y: the GEMM gate, plus bf16 rounding (2^-8
    # relative), plus E4M3 rounding (2^-4 relative, or half the smallest subnormal step s * 2^-10)
    dq = orc.e4m3_decode_array(host(yq)) * np.repeat(host(ys).astype(np.float64), 128, axis=1)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bound = 1e-2 * rms + (2.0 ** -8 + 2.0 ** -4 * (1 + 2.0 ** -8)) * np.abs(ref) + \
        np.repeat(host(ys).astype(np.float64), 128, axis=1) * 2.0 ** -10 * 1.01
    err = np.abs(dq - ref)
    say("  dequantized output codes: max err / bound = %.3f" % float((err / bound).max()))
    assert (err <= bound).all()


def test_gemm_quant_empty_and_workspace(fp8bs):
    xq = torch.empty((0, 256), dtype=torch.uint8, device="cuda")
    xs = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    wq = torch.zeros((128, 256), dtype=torch.uint8, device="cuda")
    ws = torch.ones((1, 2), dtype=torch.float32, device="cuda")
    y, yq, ys = fp8bs.fp8_block_gemm_quant(xq, xs, wq, ws)
    assert y.shape == (0, 128) and yq.shape == (0, 128) and ys.shape == (0, 1)
