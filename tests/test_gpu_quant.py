"""GPU parity of the quantizers: codes and scales bit-exact against the oracle.

Inputs are the seeded synthetic workloads (``synth``) at the shapes of the
tiny layer, the 8B-shaped dense layers, the per-step recalibration weights,
the decode activations and the MoE activations, plus ragged shapes and
special blocks, and an enumeration of every bf16 (x, amax) pair.
"""

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitexact, bf16_to_dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.lib()
    return m


ACT_SHAPES = [
    (256, 512),       # tiny layer
    (1, 128), (3, 384), (127, 256), (129, 1024), (1000, 640),  # ragged
    (1, 4096), (16, 14336), (64, 4096), (256, 14336),         # decode activations
    (8192, 4096), (8192, 14336),                               # 8B-shaped dense layers
    (65536, 2048), (65536, 768),                               # MoE rows (top-8 of 8192 tokens)
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", ACT_SHAPES, ids=lambda s: "%dx%d" % s)
def test_quant_act_parity(fp8bs, orc, shape, mode):
    M, K = shape
    say("quant_act_1x128 M=%d K=%d mode=%d" % (M, K, mode))
    x = synth.activations(M, K, seed=synth.SEED, sub=synth.SUB_X)
    q_ref, s_ref = orc.quant_act_1x128(x, mode)
    q, s = fp8bs.quant_act_1x128(bf16_to_dev(x), mode)
    assert_bitexact("codes", host(q), q_ref)
    assert_bitexact("scales", host(s), s_ref)


W_SHAPES = [
    (512, 512), (128, 128), (384, 256), (256, 1152),
    (6144, 4096), (4096, 4096), (28672, 4096), (4096, 14336),   # per-step recalibration shapes
    (1536, 2048), (2048, 768),                                  # one MoE expert
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", W_SHAPES, ids=lambda s: "%dx%d" % s)
def test_quant_w_parity(fp8bs, orc, shape, mode):
    N, K = shape
    say("quant_w_128x128 N=%d K=%d mode=%d" % (N, K, mode))
    w = synth.weights(N, K, seed=synth.SEED, sub=synth.sub_layer(0))
    q_ref, s_ref = orc.quant_w_128x128(w, mode)
    q, s = fp8bs.quant_w_128x128(bf16_to_dev(w), mode)
    assert_bitexact("codes", host(q), q_ref)
    assert_bitexact("scales", host(s), s_ref)


@pytest.mark.parametrize("mode", [0, 1])
def test_quant_w_batched_parity(fp8bs, orc, mode):
    """40 tensors of mixed shapes in one call (more than one launch's worth)."""
    shapes = [(128 * (1 + i % 5), 128 * (1 + (i * 7) % 9)) for i in range(40)]
    say("quant_w_128x128_batched %d tensors mode=%d" % (len(shapes), mode))
    ws = [synth.weights(n, k, seed=synth.SEED, sub=synth.sub_layer(i)) for i, (n, k) in enumerate(shapes)]
    outs = fp8bs.quant_w_128x128_batched([bf16_to_dev(w) for w in ws], mode)
    for i, (w, (q, s)) in enumerate(zip(ws, outs)):
        q_ref, s_ref = orc.quant_w_128x128(w, mode)
        assert_bitexact("codes[%d]" % i, host(q), q_ref)
        assert_bitexact("scales[%d]" % i, host(s), s_ref)


def _special_blocks():
    """Blocks that exercise the scale rule's edges: zeros, signed zeros, tiny
    (subnormal-scale) amax, the bf16 extremes, a lone non-zero, ties."""
    rows = []
    z = np.zeros(128, np.uint16)
    rows.append(z.copy())                                   # all +0
    rows.append(z | 0x8000)                                 # all -0
    b = z.copy(); b[17] = 0x3F80; rows.append(b)            # lone 1.0
    b = z | 0x8000; b[3] = 0xBF80; rows.append(b)          # lone -1.0 among -0
    b = np.arange(128, dtype=np.uint16) + 1; rows.append(b)            # subnormal bf16 values
    b = (np.arange(128, dtype=np.uint16) + 1) | 0x8000; rows.append(b)
    b = np.full(128, 0x0001, np.uint16); rows.append(b)                # amax = 2^-133
    b = np.full(128, 0x7F7F, np.uint16); b[::2] |= 0x8000; rows.append(b)  # +-max finite
    b = (np.arange(128, dtype=np.uint16) * 0x00FF) % 0x7F80; rows.append(b)   # spread of magnitudes
    for e in (0x0080, 0x0100, 0x0C00, 0x2000, 0x4000, 0x7000):            # one exponent range each
        g = np.random.default_rng(e)
        rows.append((g.integers(0, 0x0400, 128) + e).astype(np.uint16) | (g.integers(0, 2, 128) << 15).astype(np.uint16))
    return np.stack(rows)


@pytest.mark.parametrize("mode", [0, 1])
def test_quant_special_blocks(fp8bs, orc, mode):
    x = _special_blocks()
    x = np.concatenate([x, x[::-1]], axis=1)  # also as the second block of a row
    say("special blocks mode=%d rows=%d" % (mode, x.shape[0]))
    q_ref, s_ref = orc.quant_act_1x128(x, mode)
    q, s = fp8bs.quant_act_1x128(bf16_to_dev(x), mode)
    assert_bitexact("codes", host(q), q_ref)
    assert_bitexact("scales", host(s), s_ref)
    # the same values as 128x128 weight blocks (rows repeated to fill the tile)
    w = np.resize(x, (256, 256)).astype(np.uint16)
    qw_ref, sw_ref = orc.quant_w_128x128(w, mode)
    qw, sw = fp8bs.quant_w_128x128(bf16_to_dev(w), mode)
    assert_bitexact("w codes", host(qw), qw_ref)
    assert_bitexact("w scales", host(sw), sw_ref)


def test_quant_deterministic(fp8bs):
    x = bf16_to_dev(synth.activations(512, 2048, seed=3))
    a = fp8bs.quant_act_1x128(x, 0)
    b = fp8bs.quant_act_1x128(x, 0)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


@pytest.mark.parametrize("mode,signs", [(0, (0, 1)), (1, (0, 1))])
def test_quant_exhaustive_pairs(fp8bs, orc, mode, signs):
    """Every bf16 pair (x, amax) with 0 <= x <= amax, amax positive finite:
    amax in slot 0 of a 1x128 block, x in the other slots; both signs."""
    total = 0
    for sign in signs:
        for lo, hi in synth.pair_block_ranges(1 << 26):
            blocks = synth.pair_blocks(lo, hi, sign)
            q_ref, s_ref = orc.quant_act_1x128(blocks, mode)
            q, s = fp8bs.quant_act_1x128(bf16_to_dev(blocks), mode)
            assert_bitexact("codes amax[%#x,%#x) sign=%d" % (lo, hi, sign), host(q), q_ref)
            assert_bitexact("scales amax[%#x,%#x) sign=%d" % (lo, hi, sign), host(s), s_ref)
            total += blocks.size
    say("exhaustive pairs mode=%d: %d elements compared" % (mode, total))
