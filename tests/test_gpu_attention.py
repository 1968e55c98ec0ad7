"""GPU parity of fp8_kv_attention_decode: one query token per sequence over an
FP8 KV cache, against the oracle's fp64 attention on the same cache.

The cache is filled by the library's own quant_act_1x128 over the
[B * T, Hkv * 128] key and value rows (its codes and scales are checked bit
for bit against the oracle's quantizer: the KV-cache quantizer is the 1x128
activation quantizer).  Gate (fp32 output): max |o_gpu - o_oracle| <=
1e-3 * rms(o_oracle), a tenth of the GEMM gate, since the only rounding is
fp32 (scores from exact bf16 products, fp32 exp2 and sums); the bf16 output
must equal the round-to-nearest-even of the fp32 output bit for bit, and two
calls must be bit-identical.
"""

import math

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitexact, bf16_to_dev, host, say, to_dev

pytestmark = pytest.mark.gpu
ATT_TOL = 1e-3


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.lib()
    return m


def _case(fp8bs, orc, B, T, Hq, Hkv, lens, seed, kv_std=1.0):
    k = synth.activations(B * T, Hkv * 128, seed=seed, sub=synth.SUB_X)
    v = synth.activations(B * T, Hkv * 128, seed=seed, sub=synth.SUB_W)
    q = synth.activations(B * Hq, 128, seed=seed, sub=synth.SUB_DY)
    kq, ks = fp8bs.quant_act_1x128(bf16_to_dev(k))
    vq, vs = fp8bs.quant_act_1x128(bf16_to_dev(v))
    kq_r, ks_r = orc.quant_act_1x128(k)
    vq_r, vs_r = orc.quant_act_1x128(v)
    assert_bitexact("kq", host(kq), kq_r)
    assert_bitexact("ks", host(ks), ks_r)
    assert_bitexact("vq", host(vq), vq_r)
    assert_bitexact("vs", host(vs), vs_r)
    sh = lambda a, last: a.reshape(B, T, Hkv, *last)  # noqa: E731
    dev = dict(q=bf16_to_dev(q).view(B, Hq, 128), kq=kq.view(B, T, Hkv, 128), ks=ks.view(B, T, Hkv),
               vq=vq.view(B, T, Hkv, 128), vs=vs.view(B, T, Hkv), lens=to_dev(np.asarray(lens, np.int32)))
    ref = dict(q=q.reshape(B, Hq, 128), kq=sh(kq_r, (128,)), ks=sh(ks_r, ()), vq=sh(vq_r, (128,)),
               vs=sh(vs_r, ()), lens=np.asarray(lens, np.int32))
    return dev, ref


CASES = [
    # (name, B, T, Hq, Hkv, lens): Llama-3.1-8B heads (32 query, 8 key/value), Qwen3-30B heads (32 / 4),
    # one and two query heads per group, ragged lengths, an empty context, lengths past T (clamped),
    # contexts long enough to be split over several workgroups
    ("llama_ragged", 4, 1024, 32, 8, [1024, 700, 1, 0]),
    ("qwen_g8", 3, 300, 32, 4, [300, 17, 299]),
    ("g1", 2, 200, 4, 4, [200, 63]),
    ("g2", 2, 129, 8, 4, [129, 128]),
    ("split_long", 8, 4096, 32, 8, [4096, 4000, 2049, 513, 1, 4095, 3000, 9999]),
    # 80 sequences of one key/value head group: 7 splits per sequence, so the merge of the splits
    # takes one group of four and a tail of three
    ("splits7", 80, 2048, 4, 2, [2048 - 23 * i for i in range(80)]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: c[0])
def test_kv_attention_parity(fp8bs, orc, case):
    name, B, T, Hq, Hkv, lens = case
    sm = 1.0 / math.sqrt(128.0)
    say("fp8_kv_attention_decode %s B=%d T=%d Hq=%d Hkv=%d ws=%d" %
        (name, B, T, Hq, Hkv, fp8bs.kv_attention_workspace_size(B, T, Hq, Hkv)))
    dev, ref = _case(fp8bs, orc, B, T, Hq, Hkv, lens, seed=B * 7 + T)
    args = (dev["q"], dev["kq"], dev["ks"], dev["vq"], dev["vs"], dev["lens"], sm)
    o32 = fp8bs.fp8_kv_attention_decode(*args, out_dtype=torch.float32)
    o16 = fp8bs.fp8_kv_attention_decode(*args, out_dtype=torch.bfloat16)
    assert torch.equal(o16.view(torch.int16), o32.to(torch.bfloat16).view(torch.int16))
    assert torch.equal(o32.view(torch.int32), fp8bs.fp8_kv_attention_decode(*args, out_dtype=torch.float32)
                       .view(torch.int32))
    want = orc.kv_attention_decode(ref["q"], ref["kq"], ref["ks"], ref["vq"], ref["vs"], ref["lens"], float(np.float32(sm)))
    got = host(o32).astype(np.float64)
    assert np.isfinite(got).all()
    empty = np.clip(ref["lens"], 0, T) == 0
    assert np.all(got[empty] == 0.0)
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = float(np.abs(got - want).max())
    say("  max|err| = %.3e, rms = %.3e, max|err|/rms = %.3e" % (err, rms, err / rms))
    assert err <= ATT_TOL * rms


def test_kv_attention_peaked_scores(fp8bs, orc):
    """Large query norms: scores spread over hundreds of log2 units, so each head is
    dominated by a few tokens (the online softmax rescales many times)."""
    B, T, Hq, Hkv = 2, 777, 8, 2
    dev, ref = _case(fp8bs, orc, B, T, Hq, Hkv, [777, 400], seed=11)
    q = dev["q"] * 16
    qr = synth.f32_to_bf16_bits(synth.bf16_bits_to_f32(ref["q"]) * 16)
    assert np.array_equal(host(q.view(torch.int16)).view(np.uint16), qr)
    o = fp8bs.fp8_kv_attention_decode(q, dev["kq"], dev["ks"], dev["vq"], dev["vs"], dev["lens"], 0.125,
                                      out_dtype=torch.float32)
    want = orc.kv_attention_decode(qr, ref["kq"], ref["ks"], ref["vq"], ref["vs"], ref["lens"], 0.125)
    rms = float(np.sqrt(np.mean(want ** 2)))
    err = float(np.abs(host(o).astype(np.float64) - want).max())
    say("  peaked: max|err|/rms = %.3e" % (err / rms))
    assert err <= ATT_TOL * rms
