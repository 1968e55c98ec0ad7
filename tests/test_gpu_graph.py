"""HIP graph capture of the library's calls.

Three call sequences are captured once and replayed:
- the tiny linear layer: quant_act_1x128, quant_w_128x128 and fp8_block_gemm;
- a decode product split along K: partial sums in the caller's workspace, then a reduction launch;
- a grouped product: the tile-table launch, then the two GEMM passes.

The library issues only kernel launches: no memset, copy, allocation or synchronization. So a
captured call replays exactly what the eager call runs. Every replay must equal the eager result bit
for bit, with eager work and synchronizations between the replays and the outputs cleared before
each. After new inputs are written into the captured buffers, a replay must equal the eager call on
those new inputs.
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


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replays_equal_eager(g, outs, reps=4):
    ref = [t.clone() for t in outs]
    for r in range(reps):
        for t in outs:
            t.zero_()
        busy = torch.arange(1 << 16, device="cuda", dtype=torch.float32)
        busy = busy * 2.0  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), "replay %d: output %d differs from the eager result" % (r, i)
        del busy


def test_tiny_layer_graph(fp8bs, orc):
    M, N, K = 256, 512, 512
    say("graph: tiny layer %dx%dx%d" % (M, N, K))
    xn, wn = synth.activations(M, K), synth.weights(N, K)
    x, w = bf16_to_dev(xn), bf16_to_dev(wn)
    xq = torch.empty((M, K), dtype=torch.uint8, device="cuda")
    xs = torch.empty((M, K // 128), dtype=torch.float32, device="cuda")
    wq = torch.empty((N, K), dtype=torch.uint8, device="cuda")
    ws = torch.empty((N // 128, K // 128), dtype=torch.float32, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")

    def layer():
        fp8bs.quant_act_1x128(x, 0, out=(xq, xs))
        fp8bs.quant_w_128x128(w, 0, out=(wq, ws))
        fp8bs.fp8_block_gemm(xq, xs, wq, ws, out_dtype=torch.float32, out=y)

    layer()
    torch.cuda.synchronize()
    # the eager layer against the oracle, so that the replays are tied to it
    (xq_r, xs_r), (wq_r, ws_r) = orc.quant_act_1x128(xn, 0), orc.quant_w_128x128(wn, 0)
    assert_bitexact("xq", host(xq), xq_r)
    assert_bitexact("wq", host(wq), wq_r)
    gemm_gate("Y fp32", host(y), orc.gemm(xq_r, xs_r, wq_r, ws_r))

    g = _capture(layer)
    _replays_equal_eager(g, [xq, xs, wq, ws, y])
    # new inputs in the captured buffers: the replay reads them
    x.copy_(bf16_to_dev(synth.activations(M, K, sub=synth.SUB_X + 7)))
    w.copy_(bf16_to_dev(synth.weights(N, K, sub=synth.SUB_W + 7)))
    g.replay()
    torch.cuda.synchronize()
    replayed = [t.clone() for t in (xq, xs, wq, ws, y)]
    layer()
    torch.cuda.synchronize()
    for a, b in zip(replayed, (xq, xs, wq, ws, y)):
        assert torch.equal(a, b)


def test_split_k_decode_gemm_graph(fp8bs):
    M, N, K = 64, 4096, 4096
    say("graph: split-K GEMM %dx%dx%d" % (M, N, K))
    xq, xs = fp8bs.quant_act_1x128(bf16_to_dev(synth.activations(M, K)), 0)
    wq, ws = fp8bs.quant_w_128x128(bf16_to_dev(synth.weights(N, K)), 0)
    need = fp8bs.gemm_workspace_size(M, N, K)
    assert need > 0, "this shape is meant to be split along K"
    work = torch.empty(need, dtype=torch.uint8, device="cuda")
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def call():
        fp8bs.fp8_block_gemm(xq, xs, wq, ws, out=y, workspace=work)

    call()
    torch.cuda.synchronize()
    g = _capture(call)
    _replays_equal_eager(g, [y])


def test_grouped_gemm_graph(fp8bs):
    E, N, K = 8, 512, 256
    counts = np.array([130, 0, 257, 1, 64, 300, 129, 45], dtype=np.int64)
    offs = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    Mt = int(offs[-1])
    say("graph: grouped GEMM E=%d rows=%d N=%d K=%d" % (E, Mt, N, K))
    xq, xs = fp8bs.quant_act_1x128(bf16_to_dev(synth.activations(Mt, K)), 0)
    wq, ws = fp8bs.quant_w_128x128(bf16_to_dev(synth.weights(E * N, K)), 0)
    wq, ws = wq.view(E, N, K), ws.view(E, N // 128, K // 128)
    offs_d = torch.from_numpy(offs).to("cuda")
    work = torch.empty(max(1, fp8bs.grouped_workspace_size(E, Mt, N, K)), dtype=torch.uint8, device="cuda")
    y = torch.empty((Mt, N), dtype=torch.bfloat16, device="cuda")

    def call():
        fp8bs.fp8_block_grouped_gemm(xq, xs, wq, ws, offs_d, out=y, workspace=work)

    call()
    torch.cuda.synchronize()
    g = _capture(call)
    _replays_equal_eager(g, [y])
