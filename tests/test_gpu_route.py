"""GPU parity of the MoE dispatch quantizer (quant_act_1x128_gather): codes and
scales bit-exact against the oracle's quantization of the gathered rows, on
the MoE routing (8192 tokens, 128 experts, top-8: 65,536 rows) and on small
cases with repeated, skipped and reordered rows; indices outside the token
tensor read as zero rows."""

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
