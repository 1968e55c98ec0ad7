"""GPU parity of the MoE dispatch quantizers (quant_act_1x128_gather, and
quant_act_1x128_scatter, the same dispatch from the token side): codes and
scales bit-exact against the oracle's quantization of the gathered rows, on
the MoE routing (8192 tokens, 128 experts, top-8: 65,536 rows) and on small
cases with repeated, skipped and reordered rows; indices outside the token
tensor read as zero rows (gather); destinations outside [0, M) are skipped
and rows no destination names are left as they were (scatter)."""

import numpy as np
import pytest
import torch

import synth
from gpu_util import assert_bitexact, bf16_to_dev, dev, host, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.lib()
    return m


def _check(fp8bs, orc, x, rows, mode, name):
    q_ref, s_ref = orc.quant_act_1x128_gather(x, rows, mode)
    q, s = fp8bs.quant_act_1x128_gather(bf16_to_dev(x), torch.from_numpy(rows.astype(np.int32)).to(dev()), mode)
    assert_bitexact(name + " codes", host(q), q_ref)
    assert_bitexact(name + " scales", host(s), s_ref)


@pytest.mark.parametrize("mode", [0, 1])
def test_gather_moe_routing(fp8bs, orc, mode):
    say("quant_act_1x128_gather MoE routing T=8192 K=2048 mode=%d" % mode)
    row_token, offs = synth.moe_routing(8192, 128, 8)
    assert int(offs[-1]) == 65536
    x = synth.activations(8192, 2048)
    _check(fp8bs, orc, x, np.asarray(row_token), mode, "moe dispatch")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T, K, M", [(1, 128, 1), (5, 384, 37), (130, 640, 1000), (64, 1280, 3)])
def test_gather_small(fp8bs, orc, T, K, M, mode):
    say("quant_act_1x128_gather T=%d K=%d M=%d mode=%d" % (T, K, M, mode))
    x = synth.activations(T, K, sub=78)
    rows = np.random.default_rng(T + M).integers(0, T, M)
    _check(fp8bs, orc, x, rows, mode, "gather")


def test_gather_empty_and_out_of_range(fp8bs, orc):
    say("quant_act_1x128_gather empty and out-of-range indices")
    x = synth.activations(16, 256, sub=79)
    xd = bf16_to_dev(x)
    q, s = fp8bs.quant_act_1x128_gather(xd, torch.zeros(0, dtype=torch.int32, device=dev()))
    assert q.shape == (0, 256) and s.shape == (0, 2)
    rows = np.array([3, -1, 16, 1 << 30, 15], dtype=np.int32)
    q, s = fp8bs.quant_act_1x128_gather(xd, torch.from_numpy(rows).to(dev()))
    q, s = host(q), host(s)
    q_ref, s_ref = orc.quant_act_1x128_gather(x, np.array([3, 15]), 0)
    assert_bitexact("valid rows codes", q[[0, 4]], q_ref)
    assert_bitexact("valid rows scales", s[[0, 4]], s_ref)
    assert (q[1:4] == 0).all() and (s[1:4] == 1.0).all()  # outside [0, T): a zero row


@pytest.mark.parametrize("mode", [0, 1])
def test_scatter_moe_routing(fp8bs, orc, mode):
    """Each token quantized once and written to its 8 expert rows: the oracle's quantization of
    the gathered rows (row_token is the inverse of dest)."""
    say("quant_act_1x128_scatter MoE routing T=8192 K=2048 mode=%d" % mode)
    row_token, offs = synth.moe_routing(8192, 128, 8)
    dest = synth.moe_dest(row_token, 8192, 8)
    assert (dest >= 0).all() and np.array_equal(np.sort(dest.reshape(-1)), np.arange(65536))
    x = synth.activations(8192, 2048)
    q, s = fp8bs.quant_act_1x128_scatter(bf16_to_dev(x), torch.from_numpy(dest).to(dev()), 65536, mode)
    q_ref, s_ref = orc.quant_act_1x128_gather(x, np.asarray(row_token), mode)
    assert_bitexact("scatter codes", host(q), q_ref)
    assert_bitexact("scatter scales", host(s), s_ref)


@pytest.mark.parametrize("mode", [0, 1])
def test_scatter_partial_and_skipped(fp8bs, orc, mode):
    """Destinations outside [0, M) are skipped; rows that no destination names keep their contents."""
    say("quant_act_1x128_scatter partial cover mode=%d" % mode)
    T, K, topk, M = 40, 384, 3, 100
    g = np.random.default_rng(3)
    x = synth.activations(T, K, sub=80)
    slots = np.full(T * topk, -1, dtype=np.int32)          # 120 slots, 80 of the 100 rows named once
    slots[:80] = g.permutation(M)[:80]
    dest = g.permutation(slots).reshape(T, topk).astype(np.int32)
    dest[0, 0] = M          # past the end: skipped
    dest[1, 1] = 1 << 30
    covered = np.zeros(M, bool)
    row_of = np.full(M, -1)
    for t in range(T):
        for k in range(topk):
            d = dest[t, k]
            if 0 <= d < M:
                covered[d] = True
                row_of[d] = t
    q0 = torch.full((M, K), 0x5A, dtype=torch.uint8, device=dev())
    s0 = torch.full((M, K // 128), 7.0, dtype=torch.float32, device=dev())
    q, s = fp8bs.quant_act_1x128_scatter(bf16_to_dev(x), torch.from_numpy(dest).to(dev()), M, mode, out=(q0, s0))
    q, s = host(q), host(s)
    q_ref, s_ref = orc.quant_act_1x128_gather(x, row_of[covered], mode)
    assert_bitexact("covered codes", q[covered], q_ref)
    assert_bitexact("covered scales", s[covered], s_ref)
    assert (q[~covered] == 0x5A).all() and (s[~covered] == 7.0).all()
