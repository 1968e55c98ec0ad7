"""Pins of the oracle's gated activation (the input of the MLP's down projection).

The article ("NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
precision training") keeps non-linear functions in BF16 (section "Technical
breakthrough") and blames part of the gap to the 2x peak on quantization
kernel overhead (section "Real-world performance gains").  The oracle's
reading: h = RN_bf16((g * sigma(g)) * u) evaluated in fp64, then the 1x128
activation quantizer.  The tests tie it to things other than itself:
  - the bf16 rounding, to integer rounding of fp32 bit patterns, torch's
    float32 -> bfloat16 cast, and hand-placed midpoints, subnormals and the
    overflow boundary (values a double holds but fp32 does not, so a detour
    through fp32 would round twice and fail);
  - the gated activation, to a 60-digit decimal evaluation rounded to bf16 by
    exact rational arithmetic, and to closed-form special cases;
  - the fused quantization, to that decimal reference passed through the
    (separately pinned) activation quantizer.
"""

import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth


def _bf16_bits_from_f32_bits(b: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even of fp32 bit patterns to bf16, in integer arithmetic."""
    b = b.astype(np.uint64)
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16).astype(np.uint16)


def _rne_bf16_exact(v: Fraction) -> int:
    """bf16 payload nearest to the rational v (ties to even), exactly."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e, -126) - 7
    n = a / Fraction(2) ** qe
    r = math.floor(n)
    rem = n - r
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and r % 2 == 1):
        r += 1
    val = Fraction(r) * Fraction(2) ** qe
    if val >= Fraction(2) ** 128:
        return sign | 0x7F80
    f = np.float32(float(val))  # exact: at most 8 significant bits
    return sign | int(f.view(np.uint32) >> 16)


def _bf16_fraction(payload: int) -> Fraction:
    return Fraction(float(synth.bf16_bits_to_f32(np.array([payload], dtype=np.uint16))[0]))


def _swiglu_decimal(gp: int, up: int) -> Fraction:
    g = _bf16_fraction(gp)
    u = _bf16_fraction(up)
    with localcontext() as ctx:
        ctx.prec = 60
        gd = Decimal(g.numerator) / Decimal(g.denominator)
        sig = Decimal(1) / (Decimal(1) + (-gd).exp())
        h = gd * sig * (Decimal(u.numerator) / Decimal(u.denominator))
    return Fraction(h)


def _near_midpoint(v: Fraction, rel: float = 2.0 ** -48) -> bool:
    """True when v lies within rel (relative) of a bf16 rounding midpoint."""
    if v == 0:
        return False
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** (max(e, -126) - 7)
    n = a / q
    frac = n - math.floor(n)
    return abs(frac - Fraction(1, 2)) * q <= a * Fraction(rel)


# ---- bf16 rounding of a double ---------------------------------------------------

def test_bf16_from_double_matches_integer_rounding_of_fp32_patterns(orc):
    """Every double that is an fp32 value rounds like the integer RNE of its
    fp32 bit pattern, and like torch's float32 -> bfloat16 cast."""
    g = np.random.default_rng(11)
    bits = g.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32)
    bits = bits[(bits & 0x7F800000) != 0x7F800000]  # finite only
    vals = bits.view(np.float32)
    want = _bf16_bits_from_f32_bits(bits)
    got = np.array([orc.bf16_from_double(float(v)) for v in vals], dtype=np.uint16)
    assert np.array_equal(got, want)
    t = torch.from_numpy(vals.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, t)


@pytest.mark.parametrize("v, want", [
    (1.0, 0x3F80),
    (1.0 + 2.0 ** -8, 0x3F80),                  # midpoint of 1 and 1 + 2^-7: even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),              # midpoint of 0x3F81 and 0x3F82: even
    (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),     # just above the midpoint (fp32 cannot hold it)
    (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
    (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),
    (2.0 ** -133, 0x0001),                      # smallest subnormal
    (2.0 ** -134, 0x0000),                      # half of it: tie to even (zero)
    (2.0 ** -134 * (1 + 2.0 ** -30), 0x0001),
    (3 * 2.0 ** -134, 0x0002),                  # tie between 1 and 2 units: even
    (-(2.0 ** -134), 0x8000),
    (127 * 2.0 ** -133, 0x007F),                # largest subnormal
    (2.0 ** -126, 0x0080),                      # smallest normal
    (255 * 2.0 ** 120, 0x7F7F),                 # largest finite
    (255.5 * 2.0 ** 120, 0x7F80),               # tie past the largest finite: infinity
    (255.5 * 2.0 ** 120 * (1 - 2.0 ** -40), 0x7F7F),
    (1e300, 0x7F80),
    (-1e300, 0xFF80),
    (0.0, 0x0000),
    (-0.0, 0x8000),
])
def test_bf16_from_double_hand_values(orc, v, want):
    assert orc.bf16_from_double(v) == want
    if v != 0.0:  # (a Fraction has no signed zero)
        assert _rne_bf16_exact(Fraction(v)) == want  # the test's own exact rounding agrees


# ---- the gated activation ----------------------------------------------------------

def _pairs(n, seed):
    """Random (gate, up) bf16 payload pairs over the workload's spread and both
    tails of the logistic function."""
    g = np.random.default_rng(seed)
    gv = np.concatenate([g.standard_normal(n // 2) * 3.0, g.uniform(-120.0, 120.0, n - n // 2)])
    uv = g.standard_normal(n) * np.exp2(g.integers(-30, 30, n))
    return (synth.f32_to_bf16_bits(gv.astype(np.float32)), synth.f32_to_bf16_bits(uv.astype(np.float32)))


def test_swiglu_matches_decimal_evaluation(orc):
    """h equals the 60-digit value rounded to bf16 exactly, wherever that value
    is not within 2^-48 of a bf16 midpoint (there the fp64 evaluation decides,
    and the result must be one of the two neighbours)."""
    gp, up = _pairs(6000, 5)
    gu = np.stack([gp, up], axis=1)  # F = 1: [M, 2]
    h = orc.swiglu_bf16(gu)[:, 0]
    near = 0
    for i in range(gp.size):
        ex = _swiglu_decimal(int(gp[i]), int(up[i]))
        want = _rne_bf16_exact(ex)
        if _near_midpoint(ex):
            near += 1
            lo = _rne_bf16_exact(ex * (1 - Fraction(1, 1 << 40)))
            hi = _rne_bf16_exact(ex * (1 + Fraction(1, 1 << 40)))
            assert int(h[i]) in (lo, hi), i
        else:
            assert int(h[i]) == want, (i, hex(gp[i]), hex(up[i]), hex(h[i]), hex(want))
    assert near < gp.size // 20


@pytest.mark.parametrize("up", [0x3F80, 0xC040])  # u = 1 and u = -3
def test_swiglu_every_gate_value(orc, up):
    """Every finite bf16 gate value against the 60-digit evaluation rounded
    exactly (values within 2^-48 of a midpoint may take either neighbour).
    For g < -200 the exact |h| is below 2^-134 and rounds to a zero carrying
    the sign of g * u; signed zeros of g keep theirs."""
    p = np.arange(1 << 16, dtype=np.uint32)
    gp = p[(p & 0x7F80) != 0x7F80].astype(np.uint16)
    h = orc.swiglu_bf16(np.stack([gp, np.full_like(gp, up)], axis=1))[:, 0]
    u_neg = bool(up & 0x8000)
    gf = synth.bf16_bits_to_f32(gp)
    for i in range(gp.size):
        g_neg = bool(gp[i] & 0x8000)
        if gf[i] == 0 or gf[i] < -200:
            want = 0x8000 if g_neg != u_neg else 0x0000
            assert int(h[i]) == want, (hex(gp[i]), hex(h[i]))
            continue
        ex = _swiglu_decimal(int(gp[i]), up)
        if _near_midpoint(ex):
            lo = _rne_bf16_exact(ex * (1 - Fraction(1, 1 << 40)))
            hi = _rne_bf16_exact(ex * (1 + Fraction(1, 1 << 40)))
            assert int(h[i]) in (lo, hi), hex(gp[i])
        else:
            assert int(h[i]) == _rne_bf16_exact(ex), (hex(gp[i]), hex(h[i]), hex(_rne_bf16_exact(ex)))


def test_swiglu_fp64_reading_where_sigma_rounds_to_one(orc):
    """For g >= 40, 1 + exp(-g) == 1 in fp64, so the reading gives
    h = RN_bf16(g * u) exactly, ties (exact bf16 midpoints g * u) to even."""
    g = np.random.default_rng(3)
    gv = synth.f32_to_bf16_bits(g.uniform(40.0, 400.0, 3000).astype(np.float32))
    uv = synth.f32_to_bf16_bits((g.standard_normal(3000) * 4).astype(np.float32))
    h = orc.swiglu_bf16(np.stack([gv, uv], axis=1))[:, 0]
    ties = 0
    for i in range(gv.size):
        prod = _bf16_fraction(int(gv[i])) * _bf16_fraction(int(uv[i]))
        ties += _near_midpoint(prod, 0.0)
        assert int(h[i]) == _rne_bf16_exact(prod), i
    assert ties > 0  # the tie rule itself was exercised


def test_swiglu_special_values(orc):
    one, two, zero, mzero = 0x3F80, 0x4000, 0x0000, 0x8000
    cases = [
        ((zero, two), zero),          # silu(+0) = +0
        ((mzero, two), mzero),        # silu(-0) = -0
        ((one, zero), zero),
        ((one, mzero), mzero),
        ((0x4300, one), 0x4300),      # g = 128: h = g
        ((0xC300, one), mzero),       # g = -128: |h| ~ 128 e^-128, below the smallest subnormal
        ((0xC2C8, 0x7F00), None),     # g = -100, u = 2^127: h ~ -6.3e-4, a normal bf16
    ]
    gu = np.array([[c[0][0], c[0][1]] for c in cases], dtype=np.uint16)
    h = orc.swiglu_bf16(gu)[:, 0]
    for (inp, want), got in zip(cases, h):
        if want is None:
            want = _rne_bf16_exact(_swiglu_decimal(*inp))
            assert want & 0x7F80 not in (0, 0x7F80)
        assert int(got) == want, (inp, hex(got), hex(want))
    # silu(1) * 2 = 2 / (1 + e^-1) = 1.4621..., nearest bf16 1.4609375 (0x3FBB)
    assert int(orc.swiglu_bf16(np.array([[one, two]], dtype=np.uint16))[0, 0]) == 0x3FBB


def test_swiglu_column_layout(orc):
    """Gate columns first: swapping the halves changes the result, and each
    output column reads gate column f and up column F + f."""
    gu = synth.gate_up(4, 256, sub=90)
    h = orc.swiglu_bf16(gu)
    F = 256
    for m in range(4):
        for f in (0, 1, 127, 128, 255):
            ex = _swiglu_decimal(int(gu[m, f]), int(gu[m, F + f]))
            if not _near_midpoint(ex):
                assert int(h[m, f]) == _rne_bf16_exact(ex)
    swapped = np.concatenate([gu[:, F:], gu[:, :F]], axis=1)
    assert not np.array_equal(orc.swiglu_bf16(swapped), h)


@pytest.mark.parametrize("mode", [0, 1])
def test_swiglu_quant_is_quantizer_of_decimal_reference(orc, mode):
    """The fused form equals the activation quantizer applied to the decimal
    reference's bf16 h (blocks with a near-midpoint element skipped)."""
    M, F = 3, 384
    gu = synth.gate_up(M, F, sub=91)
    q, s = orc.swiglu_quant_1x128(gu, mode)
    assert q.shape == (M, F) and s.shape == (M, F // 128)
    href = np.empty((M, F), dtype=np.uint16)
    ok = np.ones((M, F // 128), dtype=bool)
    for m in range(M):
        for f in range(F):
            ex = _swiglu_decimal(int(gu[m, f]), int(gu[m, F + f]))
            href[m, f] = _rne_bf16_exact(ex)
            if _near_midpoint(ex):
                ok[m, f // 128] = False
    qr, sr = orc.quant_act_1x128(href, mode)
    assert ok.sum() >= ok.size - 1
    for m in range(M):
        for b in range(F // 128):
            if ok[m, b]:
                assert np.array_equal(q[m, 128 * b:128 * b + 128], qr[m, 128 * b:128 * b + 128])
                assert s[m, b].view(np.uint32) == sr[m, b].view(np.uint32)
    # and, independently of the decimal reference, the composition of the two oracle functions
    q2, s2 = orc.quant_act_1x128(orc.swiglu_bf16(gu), mode)
    assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
