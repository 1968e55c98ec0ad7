"""Pins of the oracle's attention over an FP8 KV cache (decode: one query token
per sequence).

The article ("NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8 precision
training", section "Real-world performance gains") credits an FP8 KV cache and
FP8 attention with raising the gain to about 48%; it gives no granularity.  The
oracle reads the cache as E4M3 codes with one fp32 scale per (token, head) --
quant_act_1x128 of the [tokens, heads * 128] key and value rows -- and computes
softmax(q K^T * sm_scale) V in fp64.  The pins below are closed forms and
invariants that a dropped term, a wrong sign, a wrong head mapping or a
transposed operand would break.
"""

import math

import numpy as np
import pytest

import synth

D = 128


def _cache(orc, B, T, Hkv, seed):
    k = synth.activations(B * T, Hkv * D, seed=seed, sub=synth.SUB_X)
    v = synth.activations(B * T, Hkv * D, seed=seed, sub=synth.SUB_W)
    kq, ks = orc.quant_act_1x128(k)
    vq, vs = orc.quant_act_1x128(v)
    return (kq.reshape(B, T, Hkv, D), ks.reshape(B, T, Hkv), vq.reshape(B, T, Hkv, D), vs.reshape(B, T, Hkv))


def _dequant(orc, q, s):
    return orc.e4m3_decode_array(q) * s[..., None].astype(np.float64)


def _q(B, Hq, seed):
    return synth.activations(B * Hq, D, seed=seed, sub=synth.SUB_DY).reshape(B, Hq, D)


def test_single_token_returns_its_value(orc):
    """len = 1: the softmax weight is exactly 1, so o is the dequantized value row."""
    B, T, Hq, Hkv = 2, 4, 8, 2
    kq, ks, vq, vs = _cache(orc, B, T, Hkv, seed=1)
    o = orc.kv_attention_decode(_q(B, Hq, 1), kq, ks, vq, vs, np.array([1, 1], np.int32), 0.088)
    v0 = _dequant(orc, vq[:, 0], vs[:, 0])          # [B, Hkv, D]
    for h in range(Hq):
        assert np.array_equal(o[:, h], v0[:, h // (Hq // Hkv)])


def test_zero_query_averages_values(orc):
    """q = 0: every score is 0, the weights are uniform, o is the mean of the value rows."""
    B, T, Hq, Hkv = 2, 37, 4, 4
    kq, ks, vq, vs = _cache(orc, B, T, Hkv, seed=2)
    lens = np.array([37, 20], np.int32)
    o = orc.kv_attention_decode(np.zeros((B, Hq, D), np.uint16), kq, ks, vq, vs, lens, 0.1)
    for b in range(B):
        mean = _dequant(orc, vq[b, :lens[b]], vs[b, :lens[b]]).mean(axis=0)   # [Hkv, D]
        assert np.allclose(o[b], mean, rtol=1e-13, atol=1e-13 * np.abs(mean).max())


def test_two_keys_hand_weights(orc):
    """Two keys with scores ln 3 and 0: weights 3/4 and 1/4."""
    B, T, Hq, Hkv = 1, 2, 1, 1
    kq = np.zeros((B, T, Hkv, D), np.uint8)
    kq[0, 0] = 0x38                                   # decode = 1.0
    ks = np.ones((B, T, Hkv), np.float32)
    vq = np.zeros((B, T, Hkv, D), np.uint8)
    vq[0, 0] = 0x48                                   # 4.0
    vq[0, 1] = 0xC0                                   # -2.0
    vs = np.full((B, T, Hkv), 0.5, np.float32)
    q = np.full((B, Hq, D), 0x3F80, np.uint16)        # bf16 1.0
    o = orc.kv_attention_decode(q, kq, ks, vq, vs, np.array([2], np.int32), math.log(3.0) / D)
    want = 0.75 * 4.0 * 0.5 + 0.25 * (-2.0) * 0.5      # 1.25
    assert np.allclose(o, want, rtol=1e-14, atol=0)


def test_dominant_key_selects_its_value(orc):
    """One key scores 448 * 128 above the others: exp of the gap underflows, o = that value row."""
    B, T, Hq, Hkv = 1, 50, 2, 1
    kq = np.zeros((B, T, Hkv, D), np.uint8)
    kq[0, 17] = 0x7E                                  # 448
    ks = np.ones((B, T, Hkv), np.float32)
    _, _, vq, vs = _cache(orc, B, T, Hkv, seed=3)
    q = np.full((B, Hq, D), 0x3F80, np.uint16)
    o = orc.kv_attention_decode(q, kq, ks, vq, vs, np.array([50], np.int32), 1.0)
    assert np.array_equal(o[0, 0], _dequant(orc, vq[0, 17, 0], vs[0, 17, 0]))
    # the sign matters: with the query negated, the same key is the least likely, not the most
    o2 = orc.kv_attention_decode(q | np.uint16(0x8000), kq, ks, vq, vs, np.array([50], np.int32), 1.0)
    assert not np.allclose(o2[0, 0], o[0, 0])


def test_permuting_cache_positions_is_invariant(orc):
    B, T, Hq, Hkv = 1, 64, 8, 2
    kq, ks, vq, vs = _cache(orc, B, T, Hkv, seed=4)
    q = _q(B, Hq, 4)
    lens = np.array([64], np.int32)
    o = orc.kv_attention_decode(q, kq, ks, vq, vs, lens, 0.088)
    p = np.random.default_rng(0).permutation(T)
    o2 = orc.kv_attention_decode(q, kq[:, p].copy(), ks[:, p].copy(), vq[:, p].copy(), vs[:, p].copy(), lens, 0.088)
    assert np.allclose(o, o2, rtol=1e-12, atol=1e-12 * np.abs(o).max())
    # permuting keys alone (values kept in place) changes the result
    o3 = orc.kv_attention_decode(q, kq[:, p].copy(), ks[:, p].copy(), vq, vs, lens, 0.088)
    assert not np.allclose(o, o3)


def test_positions_past_len_are_ignored_and_empty_context_is_zero(orc):
    B, T, Hq, Hkv = 3, 40, 4, 2
    kq, ks, vq, vs = _cache(orc, B, T, Hkv, seed=5)
    q = _q(B, Hq, 5)
    lens = np.array([40, 13, 0], np.int32)
    o = orc.kv_attention_decode(q, kq, ks, vq, vs, lens, 0.1)
    kq2, vq2 = kq.copy(), vq.copy()
    kq2[1, 13:] ^= 0x55
    vq2[1, 13:] = 0x7E
    o2 = orc.kv_attention_decode(q, kq2, ks, vq2, vs, lens, 0.1)
    assert np.array_equal(o[1], o2[1])
    assert np.all(o[2] == 0.0)
    # lengths beyond the cache are clamped to T
    o3 = orc.kv_attention_decode(q, kq, ks, vq, vs, np.array([99, 13, -5], np.int32), 0.1)
    assert np.array_equal(o3, o)


def test_grouped_query_heads_read_their_kv_head(orc):
    """Query head h uses key/value head h // (Hq / Hkv): equal to the single-head call on that slice."""
    B, T, Hq, Hkv = 2, 30, 8, 2
    kq, ks, vq, vs = _cache(orc, B, T, Hkv, seed=6)
    q = _q(B, Hq, 6)
    lens = np.array([30, 22], np.int32)
    o = orc.kv_attention_decode(q, kq, ks, vq, vs, lens, 0.09)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        o1 = orc.kv_attention_decode(np.ascontiguousarray(q[:, h:h + 1]), np.ascontiguousarray(kq[:, :, g:g + 1]),
                                     np.ascontiguousarray(ks[:, :, g:g + 1]), np.ascontiguousarray(vq[:, :, g:g + 1]),
                                     np.ascontiguousarray(vs[:, :, g:g + 1]), lens, 0.09)
        assert np.array_equal(o[:, h], o1[:, 0])
    # and not the other head
    assert not np.allclose(o[:, 0], o[:, Hq - 1])


def test_scale_factors_fold_into_scores_and_values(orc):
    """Doubling every key scale equals doubling sm_scale; doubling every value scale doubles o."""
    B, T, Hq, Hkv = 1, 25, 2, 1
    kq, ks, vq, vs = _cache(orc, B, T, Hkv, seed=7)
    q = _q(B, Hq, 7)
    lens = np.array([25], np.int32)
    o = orc.kv_attention_decode(q, kq, ks, vq, vs, lens, 0.05)
    assert np.allclose(orc.kv_attention_decode(q, kq, ks * 2, vq, vs, lens, 0.05),
                       orc.kv_attention_decode(q, kq, ks, vq, vs, lens, 0.1), rtol=1e-13, atol=0)
    assert np.array_equal(orc.kv_attention_decode(q, kq, ks, vq, vs * 2, lens, 0.05), 2 * o)
