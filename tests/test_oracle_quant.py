"""Pins of the oracle's block scales and quantizers.

The article ("NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8 precision
training") fixes the blocking in section "Technical breakthrough" (1x128 for
activations, 128x128 for weights, E4M3) and names power-of-2 scaling factors
as an option in its closing section.  The amax/448 rule, the zero-block
convention and the rounding of the quotient are readings stated in the
oracle's source; the tests below tie them to closed forms, invariants, brute
force and torch's own fp32 division and float8 cast.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth

ALL_POS_BF16 = np.arange(1, 0x7F80, dtype=np.uint16)  # every positive finite bf16 payload


def _f32(bits):
    return synth.bf16_bits_to_f32(bits)


# ---- scales -------------------------------------------------------------------

def test_exact_scale_is_ieee_division_and_amax_maps_to_448(orc):
    """For every positive finite bf16 amax: s == fp32(amax)/448 (numpy's IEEE
    division) and the amax element itself encodes to +-448 (0x7E / 0xFE)."""
    n = ALL_POS_BF16.size
    assert n == 32639
    blocks = np.zeros((n, 128), dtype=np.uint16)
    blocks[:, 0] = ALL_POS_BF16
    blocks[:, 1] = ALL_POS_BF16 | 0x8000  # -amax in the same block
    q, s = orc.quant_act_1x128(blocks, orc.SCALE_EXACT)
    amax = _f32(ALL_POS_BF16)
    assert np.array_equal(s[:, 0].view(np.uint32), (amax / np.float32(448.0)).view(np.uint32))
    assert (q[:, 0] == 0x7E).all()
    assert (q[:, 1] == 0xFE).all()
    assert (q[:, 2:] == 0).all()


def test_pow2_scale_is_least_power_of_two(orc):
    """POW2: s = 2^k, the least k with amax <= 448 * 2^k, checked exactly with
    rationals for every positive finite bf16 amax."""
    blocks = np.zeros((ALL_POS_BF16.size, 128), dtype=np.uint16)
    blocks[:, 5] = ALL_POS_BF16
    q, s = orc.quant_act_1x128(blocks, orc.SCALE_POW2)
    s = s[:, 0]
    amax = _f32(ALL_POS_BF16)
    mant, _ = np.frexp(s.astype(np.float64))
    assert (mant == 0.5).all(), "every POW2 scale must be a power of two"
    for a, sc in zip(amax.tolist()[::37] + amax.tolist()[-50:], s.tolist()[::37] + s.tolist()[-50:]):
        A, S = Fraction(a), Fraction(sc)
        assert A <= 448 * S and A > 448 * S / 2, (a, sc)
    # vectorised form of the same bounds (exact in fp64: powers of two times 448)
    s64 = s.astype(np.float64)
    a64 = amax.astype(np.float64)
    assert (a64 <= 448.0 * s64).all() and (a64 > 224.0 * s64).all()
    # amax / s lies in (224, 448] -> the amax element takes a code in 0x76..0x7E
    assert ((q[:, 5] >= 0x76) & (q[:, 5] <= 0x7E)).all()


def test_zero_and_signed_zero_blocks(orc):
    x = np.zeros((3, 256), dtype=np.uint16)
    x[1, :] = 0x8000  # -0 everywhere
    x[2, 128:] = 0x3F80  # +1.0 in the second block only
    for mode in (orc.SCALE_EXACT, orc.SCALE_POW2):
        q, s = orc.quant_act_1x128(x, mode)
        assert (s[0] == 1.0).all() and (s[1] == 1.0).all() and s[2, 0] == 1.0
        assert (q[0] == 0x00).all() and (q[1] == 0x80).all() and (q[2, :128] == 0).all()
        # 1.0 / s is 448 (EXACT) or 256 (POW2: s = 2^-8, the least power of two >= 1/448)
        assert (q[2, 128:] == (0x7E if mode == orc.SCALE_EXACT else 0x78)).all()
        assert s[2, 1] == (np.float32(1.0) / np.float32(448.0) if mode == orc.SCALE_EXACT else 1.0 / 256)
    w = np.zeros((256, 128), dtype=np.uint16)
    w[200, 7] = 0xC000  # -2.0 in block (1, 0)
    q, s = orc.quant_w_128x128(w, orc.SCALE_EXACT)
    assert s[0, 0] == 1.0 and (q[:128] == 0).all()
    assert q[200, 7] == 0xFE and np.count_nonzero(q[128:]) == 1


# ---- brute force on tiny shapes --------------------------------------------------

def _mag(c):
    e, m = c >> 3, c & 7
    return Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)


_MAGS = [_mag(c) for c in range(0x7F)]


def _brute_code(q32: float) -> int:
    sign = 0x80 if math.copysign(1.0, q32) < 0 else 0
    a = Fraction(abs(q32))
    best = min(range(0x7F), key=lambda c: (abs(a - _MAGS[c]), c & 1))
    return sign | best


def _brute_quant_block(vals_f32: np.ndarray, mode: int, sample=None):
    amax = Fraction(0)
    for v in vals_f32.tolist():
        amax = max(amax, abs(Fraction(v)))
    if amax == 0:
        s = np.float32(1.0)
    elif mode == 0:
        s = np.float32(float(amax)) / np.float32(448.0)
    else:
        k = 0
        while amax > 448 * Fraction(2) ** k:
            k += 1
        while amax <= 448 * Fraction(2) ** (k - 1):
            k -= 1
        s = np.float32(2.0 ** k)
    vals = vals_f32 if sample is None else vals_f32[sample]
    codes = [_brute_code(float(np.float32(v) / s)) for v in vals.tolist()]
    return codes, s


@pytest.mark.parametrize("shape", [(1, 128), (3, 256), (2, 384)])
@pytest.mark.parametrize("mode", [0, 1])
def test_quant_act_bruteforce(orc, shape, mode):
    M, K = shape
    x = synth.activations(M, K, seed=11, sub=M * 1000 + K)
    x[0, 3] = 0x8000  # a -0
    q, s = orc.quant_act_1x128(x, mode)
    xf = _f32(x)
    for m in range(M):
        for kb in range(K // 128):
            codes, sc = _brute_quant_block(xf[m, kb * 128:(kb + 1) * 128], mode)
            assert s[m, kb] == sc
            assert q[m, kb * 128:(kb + 1) * 128].tolist() == codes


@pytest.mark.parametrize("shape", [(128, 128), (256, 128)])
@pytest.mark.parametrize("mode", [0, 1])
def test_quant_w_bruteforce(orc, shape, mode):
    N, K = shape
    w = synth.weights(N, K, seed=12, sub=N + K)
    q, s = orc.quant_w_128x128(w, mode)
    wf = _f32(w)
    for nb in range(N // 128):
        tile = wf[nb * 128:(nb + 1) * 128, :128].reshape(-1)
        # amax over the whole tile; codes brute-forced on 3000 positions, amax element included
        pick = np.unique(np.concatenate([np.random.default_rng(nb).choice(16384, 3000, replace=False),
                                         [int(np.argmax(np.abs(tile)))]]))
        codes, sc = _brute_quant_block(tile, mode, sample=pick)
        assert s[nb, 0] == sc
        assert q[nb * 128:(nb + 1) * 128, :128].reshape(-1)[pick].tolist() == codes


# ---- torch's fp32 division and float8 cast as an independent route ---------------

@pytest.mark.parametrize("mode", [0, 1])
def test_quant_matches_torch_route(orc, mode):
    """codes == torch.float8_e4m3fn(fp32(x) / s) with torch's own amax and
    division; every quotient is within 448 * (1 + 2^-23) < 464, where torch's
    cast coincides with saturating round-to-nearest-even."""
    x = synth.activations(64, 1024, seed=13)
    q, s = orc.quant_act_1x128(x, mode)
    xt = torch.from_numpy(_f32(x)).view(64, 8, 128)
    amax = xt.abs().amax(dim=2)
    if mode == 0:
        st = amax / 448.0
    else:
        st = torch.from_numpy(s)  # the power-of-two choice is pinned separately above
        assert torch.all(amax <= 448.0 * st) and torch.all(amax > 224.0 * st)
    assert torch.equal(torch.from_numpy(s).view(torch.int32), st.view(torch.int32))
    qt = (xt / st[:, :, None]).to(torch.float8_e4m3fn).view(torch.uint8).reshape(64, 1024)
    assert np.array_equal(qt.numpy(), q)


# ---- invariants -----------------------------------------------------------------

@pytest.mark.parametrize("mode", [0, 1])
def test_sign_equivariance(orc, mode):
    x = synth.activations(32, 512, seed=14)
    q, s = orc.quant_act_1x128(x, mode)
    qn, sn = orc.quant_act_1x128(x ^ np.uint16(0x8000), mode)
    assert np.array_equal(qn, q ^ np.uint8(0x80)) and np.array_equal(s, sn)
    w = synth.weights(256, 256, seed=15)
    q, s = orc.quant_w_128x128(w, mode)
    qn, sn = orc.quant_w_128x128(w ^ np.uint16(0x8000), mode)
    assert np.array_equal(qn, q ^ np.uint8(0x80)) and np.array_equal(s, sn)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("j", [-20, -3, 5, 30])
def test_power_of_two_equivariance(orc, mode, j):
    """quant(2^j X) = (same codes, 2^j s) away from under/overflow."""
    x = synth.activations(16, 512, seed=16)
    xs = synth.f32_to_bf16_bits(_f32(x) * np.float32(2.0 ** j))  # exact scaling
    q, s = orc.quant_act_1x128(x, mode)
    q2, s2 = orc.quant_act_1x128(xs, mode)
    assert np.array_equal(q, q2)
    assert np.array_equal(s2, (s * np.float32(2.0 ** j)))


def test_row_permutation_equivariance(orc):
    x = synth.activations(64, 256, seed=17)
    perm = np.random.default_rng(3).permutation(64)
    q, s = orc.quant_act_1x128(x)
    qp, sp = orc.quant_act_1x128(x[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])


@pytest.mark.parametrize("mode", [0, 1])
def test_weight_transpose_symmetry(orc, mode):
    w = synth.weights(256, 384, seed=18)
    q, s = orc.quant_w_128x128(w, mode)
    qt, st = orc.quant_w_128x128(np.ascontiguousarray(w.T), mode)
    assert np.array_equal(qt, q.T) and np.array_equal(st, s.T)


def test_weight_tile_equals_one_flat_block(orc):
    """A 128x128 weight block is one block of 16384 values: its codes equal the
    1x128 quantizer's when every row of the tile shares the tile's amax."""
    w = synth.weights(128, 128, seed=19)
    q, s = orc.quant_w_128x128(w)
    amax_bits = np.max(w & 0x7FFF)
    w2 = w.copy()
    w2[:, 0] = amax_bits  # every row now holds the tile's amax in column 0
    q2w, s2w = orc.quant_w_128x128(w2)
    q2a, s2a = orc.quant_act_1x128(w2)
    assert (s2a == s2w[0, 0]).all() and s2w[0, 0] == s[0, 0]
    assert np.array_equal(q2a, q2w)
    assert np.array_equal(q2w[:, 1:], q[:, 1:])


@pytest.mark.parametrize("mode", [0, 1])
def test_dequant_error_bound(orc, mode):
    """|decode(q) - x/s| <= half an E4M3 spacing at |x/s| (+ the fp32 rounding
    of the quotient): the result lies within the format's rounding bound."""
    x = synth.activations(64, 1024, seed=20)
    q, s = orc.quant_act_1x128(x, mode)
    xf = _f32(x).astype(np.float64).reshape(64, 8, 128)
    t = xf / s.astype(np.float64)[:, :, None]
    d = orc.e4m3_decode_array(q).reshape(64, 8, 128)
    at = np.abs(t)
    e = np.floor(np.log2(np.maximum(at, 2.0 ** -6)))
    half_spacing = 2.0 ** (e - 4)
    assert (np.abs(d - t) <= half_spacing + at * 2.0 ** -23).all()
    assert np.abs(d).max() <= 448.0


def test_pow2_round_trip(orc):
    """POW2: decode(q) * s is exact and fits bf16; quantizing it again returns
    (q, s) whenever the block's largest code magnitude is above 224."""
    x = synth.activations(32, 512, seed=21)
    q, s = orc.quant_act_1x128(x, orc.SCALE_POW2)
    d = orc.e4m3_decode_array(q).reshape(32, 4, 128) * s.astype(np.float64)[:, :, None]
    d32 = d.astype(np.float32)
    assert np.array_equal(d32.astype(np.float64), d)
    bf = synth.f32_to_bf16_bits(d32.reshape(32, 512))
    assert np.array_equal(_f32(bf).astype(np.float64).reshape(d.shape), d)
    q2, s2 = orc.quant_act_1x128(bf, orc.SCALE_POW2)
    keep = (np.abs(orc.e4m3_decode_array(q)).reshape(32, 4, 128).max(axis=2) > 224)
    assert keep.mean() > 0.9
    assert np.array_equal(s2[keep], s[keep])
    assert np.array_equal(q2.reshape(32, 4, 128)[keep], q.reshape(32, 4, 128)[keep])


def test_subnormal_scale_blocks(orc):
    """Tiny blocks (amax below 448 * 2^-126) get subnormal scales that are kept,
    and the amax element still maps to 448 (EXACT) / a code in 0x76..0x7E (POW2)."""
    tiny = np.array([0x0001, 0x0003, 0x0040, 0x007F, 0x0080, 0x0100, 0x0200], dtype=np.uint16)
    blocks = np.zeros((tiny.size, 128), dtype=np.uint16)
    blocks[:, 0] = tiny
    blocks[:, 1] = tiny // 2
    q, s = orc.quant_act_1x128(blocks, orc.SCALE_EXACT)
    assert (s[:, 0] > 0).all() and (s[:, 0] < np.float32(2.0 ** -126)).any()
    assert (q[:, 0] == 0x7E).all()
    qp, sp = orc.quant_act_1x128(blocks, orc.SCALE_POW2)
    assert ((qp[:, 0] >= 0x76) & (qp[:, 0] <= 0x7E)).all()


@pytest.mark.parametrize("mode", [0, 1])
def test_quant_act_gather_equals_quantize_then_gather(orc, mode):
    """The 1x128 blocks lie along rows, so quantizing the gathered rows equals
    gathering the rows' codes and scales (the MoE dispatch reading), with
    repeated, skipped and reordered rows."""
    x = synth.activations(64, 384, sub=77)
    g = np.random.default_rng(5)
    rows = np.concatenate([g.integers(0, 64, 300), [0, 63, 63, 0]]).astype(np.int32)
    q, s = orc.quant_act_1x128_gather(x, rows, mode)
    q0, s0 = orc.quant_act_1x128(x, mode)
    assert np.array_equal(q, q0[rows]) and np.array_equal(s.view(np.uint32), s0[rows].view(np.uint32))
    q1, s1 = orc.quant_act_1x128_gather(x, np.zeros(0, dtype=np.int32), mode)
    assert q1.shape == (0, 384) and s1.shape == (0, 3)
    with pytest.raises(ValueError):
        orc.quant_act_1x128_gather(x, np.array([64], dtype=np.int32), mode)
