"""GPU test of fp8_block_grouped_gemm_noalloc, the grouped GEMM that allocates
nothing (its row-tile tables live in the library's static device array).

Called through the C ABI with caller-allocated outputs and compared with
fp8_block_grouped_gemm (same kernels: bit-identical) and with the oracle (the
GEMM gate), on two calls in a row, the second with a smaller input, so that
the second call runs on the tables the first one left in the array.
"""

import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16_to_dev, gemm_gate, host, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp8bs():
    import block_scaled_fp8_x128_amd as m
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    m.lib()
    return m


def _case(fp8bs, orc, counts, N, K, seed):
    offs = synth.offsets_from_counts(counts)
    M, E = int(offs[-1]), len(counts)
    x = synth.activations(max(M, 1), K, seed=synth.SEED, sub=synth.SUB_X + seed)[:M]
    w = synth.expert_weights(E, N, K, seed=synth.SEED, sub=synth.SUB_W + seed)
    xq, xs = fp8bs.quant_act_1x128(bf16_to_dev(x))
    wq, ws = fp8bs.quant_w_128x128(bf16_to_dev(w.reshape(E * N, K)))
    wq, ws = wq.view(E, N, K), ws.view(E, N // 128, K // 128)
    xq_r, xs_r = orc.quant_act_1x128(x)
    wq_r, ws_r = orc.quant_w_128x128(w.reshape(E * N, K))
    ref = orc.grouped_gemm_full(xq_r, xs_r, wq_r.reshape(E, N, K), ws_r.reshape(E, N // 128, K // 128), offs)
    return xq, xs, wq, ws, to_dev(offs), M, E, ref


def _noalloc(fp8bs, xq, xs, wq, ws, offs, M, E, N, K, out_dtype):
    y = torch.full((M, N), float("nan"), dtype=out_dtype, device=xq.device)
    code = fp8bs.OUT_FP32 if out_dtype == torch.float32 else fp8bs.OUT_BF16
    p = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    st = fp8bs.lib().fp8_block_grouped_gemm_noalloc(
        p(xq), p(xs), p(wq), p(ws), p(offs), E, M, N, K, p(y), code,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, fp8bs.status_string(st)
    return y


# first call: the MoE gate+up shape's expert count with ragged groups; second: fewer rows and
# experts (its tables are shorter than what the first call left in the array); then a shape whose
# N is not a multiple of 256 (the 128x128 kernel, which uses no tables)
CALLS = [
    ([700, 0, 129, 1, 513, 300, 64, 0, 257] * 4, 512, 1024),
    ([5, 0, 129, 1, 64], 256, 384),
    ([33, 7, 0, 90], 384, 256),
]


def test_noalloc_matches_workspace_entry(fp8bs, orc):
    for i, (counts, N, K) in enumerate(CALLS):
        say("fp8_block_grouped_gemm_noalloc call %d: E=%d M_total=%d N=%d K=%d" % (i, len(counts), sum(counts), N, K))
        xq, xs, wq, ws, offs, M, E, ref = _case(fp8bs, orc, counts, N, K, seed=i)
        for dt in (torch.float32, torch.bfloat16):
            y_na = _noalloc(fp8bs, xq, xs, wq, ws, offs, M, E, N, K, dt)
            y_ws = fp8bs.fp8_block_grouped_gemm(xq, xs, wq, ws, offs, out_dtype=dt)
            torch.cuda.synchronize()
            bits = torch.int32 if dt == torch.float32 else torch.int16
            assert torch.equal(y_na.view(bits), y_ws.view(bits)), "call %d %s differs" % (i, dt)
            if dt == torch.float32:
                gemm_gate("Y fp32 noalloc call %d" % i, host(y_na), ref)


def test_noalloc_rejects_oversize_before_launch(fp8bs):
    """A problem whose tables exceed the array: SCRATCH_TOO_SMALL, nothing written."""
    E, N, K = 1, 256, 256
    cap = fp8bs.NOALLOC_SCRATCH_BYTES
    m_big = ((cap - 16) // 16 - 2 * E) * 256 + 1
    assert fp8bs.grouped_workspace_size(E, m_big, N, K) > cap
    z = torch.zeros(16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(z.data_ptr())
    st = fp8bs.lib().fp8_block_grouped_gemm_noalloc(p, p, p, p, p, E, m_big, N, K, p, 0,
                                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == fp8bs.STATUS_SCRATCH_TOO_SMALL
    torch.cuda.synchronize()
    assert int(z.sum()) == 0
