"""GPU parity of the fused gated activation + 1x128 quantizer (swiglu_quant_1x128).

Codes and scales must be bit-exact against the oracle (h rounded to bf16 from
its fp64 evaluation, then the activation quantizer), on the seeded gate+up
outputs at the MoE shape (65,536 routed rows, expert FFN 768) and the
8B-shaped dense MLP (8192 tokens, FFN 14336), on ragged shapes, on every
finite bf16 gate value, and on special values that take the kernel's fp64
path (zeros, subnormals, the far negative tail, bf16 rounding midpoints).
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


SHAPES = [
    (1, 128), (3, 384), (5, 256), (127, 640), (129, 1280),   # ragged and small
    (256, 768), (1024, 1536),
    (65536, 768),                                           # MoE: 8192 tokens top-8, expert FFN 768
    (8192, 14336),                                          # 8B-shaped dense MLP
]


def _check(fp8bs, orc, gu, mode, name):
    q_ref, s_ref = orc.swiglu_quant_1x128(gu, mode)
    q, s = fp8bs.swiglu_quant_1x128(bf16_to_dev(gu), mode)
    assert_bitexact(name + " codes", host(q), q_ref)
    assert_bitexact(name + " scales", host(s), s_ref)


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "%dx%d" % s)
def test_swiglu_quant_parity(fp8bs, orc, shape, mode):
    M, F = shape
    say("swiglu_quant_1x128 M=%d F=%d mode=%d" % (M, F, mode))
    _check(fp8bs, orc, synth.gate_up(M, F), mode, "swiglu_quant")


def _finite_bf16_payloads():
    p = np.arange(1 << 16, dtype=np.uint32)
    return p[(p & 0x7F80) != 0x7F80].astype(np.uint16)  # 65,280 finite payloads, both signs


@pytest.mark.parametrize("mode", [0, 1])
def test_swiglu_quant_every_gate_value(fp8bs, orc, mode):
    """Every finite bf16 gate value, each with up values of magnitude in [2^-8, 1)
    (so |h| <= |g| stays in range): 51 rows x 1280 columns."""
    say("swiglu_quant_1x128 every gate value, mode=%d" % mode)
    g = _finite_bf16_payloads()
    assert g.size == 51 * 1280
    rng = np.random.default_rng(21)
    for rep in range(3):
        gp = rng.permutation(g).reshape(51, 1280)
        mag = np.exp2(rng.uniform(-8.0, 0.0, gp.shape)).astype(np.float32)
        sign = np.where(rng.random(gp.shape) < 0.5, -1.0, 1.0).astype(np.float32)
        up = synth.f32_to_bf16_bits(mag * sign)
        _check(fp8bs, orc, np.concatenate([gp, up], axis=1), mode, "every gate, pass %d" % rep)


@pytest.mark.parametrize("mode", [0, 1])
def test_swiglu_quant_special_values(fp8bs, orc, mode):
    """Values that leave the fp32 fast path: signed zeros, subnormal gates and
    ups, the far negative tail (g <= -64, where exp(-g) leaves fp32), results
    below 2^-64, and products g * u that are exact bf16 midpoints for large g
    (sigma(g) rounds to 1 in fp32 and the fp64 evaluation decides)."""
    say("swiglu_quant_1x128 special values, mode=%d" % mode)
    rng = np.random.default_rng(22)
    F = 512
    rows = []

    def f2b(a):
        return synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))

    # 1: zeros of both signs against random ups, and random gates against zero ups
    z = np.where(rng.random(F) < 0.5, 0x0000, 0x8000).astype(np.uint16)
    rows.append(np.concatenate([z, f2b(rng.standard_normal(F))]))
    rows.append(np.concatenate([f2b(rng.standard_normal(F) * 3), z]))
    # 2: subnormal gates and subnormal ups
    sub = rng.integers(1, 0x80, F).astype(np.uint16) | np.where(rng.random(F) < 0.5, 0, 0x8000).astype(np.uint16)
    rows.append(np.concatenate([sub, f2b(rng.standard_normal(F) * 1e30)]))
    rows.append(np.concatenate([f2b(rng.standard_normal(F) * 3), sub]))
    # 3: the negative tail, with ups large enough to keep h representable
    rows.append(np.concatenate([f2b(rng.uniform(-140.0, -60.0, F)), f2b(rng.standard_normal(F) * 1e30)]))
    rows.append(np.concatenate([f2b(rng.uniform(-90.0, -16.0, F)), f2b(rng.standard_normal(F))]))
    # 4: large gates times ups whose products are exact bf16 midpoints
    # (g = 3 * 2^k, u = 1 + odd/128: the product's significand is 3 * odd, a 9-bit
    # odd number -- an exact midpoint -- whenever it is below 512; for g = 24
    # sigma(g) rounds to 1 in fp32 only, for g >= 48 in fp64 as well)
    gl = f2b(3.0 * np.exp2(rng.integers(3, 8, F)) * np.where(rng.random(F) < 0.5, -1.0, 1.0))
    ul = f2b(1.0 + (2 * rng.integers(0, 64, F) + 1) / 128.0)
    rows.append(np.concatenate([gl, ul]))
    # 5: tiny gates (|g| < 2^-64) and tiny results
    rows.append(np.concatenate([f2b(rng.standard_normal(F) * 1e-25), f2b(rng.standard_normal(F) * 1e-15)]))
    gu = np.stack(rows).astype(np.uint16)
    _check(fp8bs, orc, gu, mode, "special")


def _midpoint_distance_units(h):
    """Distance of float64 values to the nearest bf16 rounding midpoint, in units
    of the fp32 spacing at each value (normal fp32 range only)."""
    h = np.abs(h)
    e = np.floor(np.log2(h))
    unit = np.exp2(e - 23)                  # fp32 spacing in [2^e, 2^(e+1))
    half = np.exp2(e - 8)                   # half the bf16 spacing there
    r = np.mod(h, 2 * half)                 # position within a bf16 interval
    return np.abs(r - half) / unit


@pytest.mark.parametrize("mode", [0, 1])
def test_swiglu_quant_near_the_fp64_window(fp8bs, orc, mode):
    """Elements whose value lies 16 to 64 fp32 units from a bf16 midpoint: the
    fp32 path alone decides their rounding (the fp64 recompute covers 16 and
    less), so these check its error bound where it matters."""
    say("swiglu_quant_1x128 near the fp64 window, mode=%d" % mode)
    rng = np.random.default_rng(23)
    n = 1 << 22
    g = synth.f32_to_bf16_bits((rng.standard_normal(n) * 4).astype(np.float32))
    u = synth.f32_to_bf16_bits((rng.standard_normal(n) * np.exp2(rng.integers(-20, 20, n))).astype(np.float32))
    gf = synth.bf16_bits_to_f32(g).astype(np.float64)
    uf = synth.bf16_bits_to_f32(u).astype(np.float64)
    with np.errstate(over="ignore", divide="ignore", invalid="ignore"):
        h = (gf / (1.0 + np.exp(-gf))) * uf
        d = _midpoint_distance_units(h)
    pick = (gf >= -64) & (np.abs(h) >= 2.0 ** -100) & (np.abs(h) < 2.0 ** 100) & (d > 16) & (d <= 64)
    F = 1280
    k = (int(pick.sum()) // F) * F
    assert k >= 2 * F, int(pick.sum())
    gp, up = g[pick][:k].reshape(-1, F), u[pick][:k].reshape(-1, F)
    _check(fp8bs, orc, np.concatenate([gp, up], axis=1), mode, "near the window (%d elements)" % k)


def test_swiglu_quant_empty_and_errors(fp8bs):
    say("swiglu_quant_1x128 empty and errors")
    lib = fp8bs.lib()
    e = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = fp8bs.swiglu_quant_1x128(e)
    assert q.shape == (0, 128) and s.shape == (0, 1)
    gu = torch.zeros((2, 256), dtype=torch.bfloat16, device="cuda")
    hq = torch.empty((2, 128), dtype=torch.uint8, device="cuda")
    hs = torch.empty((2, 1), dtype=torch.float32, device="cuda")
    assert lib.swiglu_quant_1x128(gu.data_ptr(), 2, 128, hq.data_ptr(), hs.data_ptr(), 2, None) == 1
    assert lib.swiglu_quant_1x128(gu.data_ptr(), 2, 64, hq.data_ptr(), hs.data_ptr(), 0, None) == 2
    assert lib.swiglu_quant_1x128(gu.data_ptr() + 2, 2, 128, hq.data_ptr(), hs.data_ptr(), 0, None) == 1
    assert lib.swiglu_quant_1x128(gu.data_ptr(), 2, 128, hq.data_ptr(), hs.data_ptr(), 0, None) == 0
    torch.cuda.synchronize()
    assert (hq.cpu() == 0).all() and (hs.cpu() == 1.0).all()  # an all-zero block: codes 0, scale 1
