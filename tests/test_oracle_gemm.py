"""Pins of the oracle's block-scaled GEMM and grouped (MoE) GEMM.

The article ("NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8 precision
training", section "Technical breakthrough") says linear layers run FP8 math on
the block-quantized operands; the MoE form follows its Qwen3-30B (mixture of
experts) result in section "Real-world performance gains".  The oracle sums
each 128-wide K block exactly and applies the two fp32 scales per block; the
tests tie that to the closed form (an fp64 matmul of the dequantized operands),
to exact integer matmuls and to the per-expert decomposition.
"""

import numpy as np
import pytest

import synth


def _dequant_rows(orc, q, s):
    """decode(q) * s with s broadcast over 1x128 blocks (activation layout)."""
    d = orc.e4m3_decode_array(q)
    return d * np.repeat(s.astype(np.float64), 128, axis=1)


def _dequant_tiles(orc, q, s):
    """decode(q) * s with s broadcast over 128x128 blocks (weight layout)."""
    d = orc.e4m3_decode_array(q)
    return d * np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)


def _operands(orc, M, N, K, seed, mode=0):
    x = synth.activations(M, K, seed=seed)
    w = synth.weights(N, K, seed=seed, sub=synth.SUB_W)
    xq, xs = orc.quant_act_1x128(x, mode)
    wq, ws = orc.quant_w_128x128(w, mode)
    return xq, xs, wq, ws


@pytest.mark.parametrize("shape", [(256, 512, 512), (256, 256, 512), (200, 384, 640), (1, 128, 128), (130, 256, 1024)])
@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_equals_matmul_of_dequantized(orc, shape, mode):
    M, N, K = shape
    xq, xs, wq, ws = _operands(orc, M, N, K, seed=M + N + K, mode=mode)
    y = orc.gemm(xq, xs, wq, ws)
    ref = _dequant_rows(orc, xq, xs) @ _dequant_tiles(orc, wq, ws).T
    rms = np.sqrt(np.mean(ref ** 2))
    assert rms > 0
    assert np.max(np.abs(y - ref)) <= 1e-12 * rms * np.sqrt(K)
    # the same closed form with the operand order swapped is a different matrix
    if M == N:
        assert np.max(np.abs(y - ref.T)) > 1e-3 * rms


@pytest.mark.parametrize("mode", [0, 1])
def test_data_gradient_from_transposed_weight_blocks(orc, mode):
    """dX = dY W: the oracle's GEMM of quant_act(dY) with the quantization of
    W^T equals the fp64 product dequant(dY) @ dequant(W) -- W's own blocks,
    untransposed -- since a 128x128 block and its transpose share amax and scale."""
    M, N, K = 130, 384, 256
    dy = synth.activations(M, N, seed=7, sub=synth.SUB_DY)
    w = synth.weights(N, K, seed=7, sub=synth.SUB_W)
    dyq, dys = orc.quant_act_1x128(dy, mode)
    wqt, wst = orc.quant_w_128x128(np.ascontiguousarray(w.T), mode)
    dx = orc.gemm(dyq, dys, wqt, wst)
    wq, ws = orc.quant_w_128x128(w, mode)
    ref = _dequant_rows(orc, dyq, dys) @ _dequant_tiles(orc, wq, ws)
    rms = np.sqrt(np.mean(ref ** 2))
    assert dx.shape == (M, K) and rms > 0
    assert np.max(np.abs(dx - ref)) <= 1e-12 * rms * np.sqrt(N)


def _dequant_row_scaled(orc, q, s):
    """decode(q) * s with s [R, K/128] broadcast over each row's 1x128 blocks."""
    return orc.e4m3_decode_array(q) * np.repeat(s.astype(np.float64), 128, axis=1)


@pytest.mark.parametrize("mode", [0, 1])
def test_weight_gradient_closed_form(orc, mode):
    """dW = dY^T X from quant_act_1x128_t of both: the oracle's 1x128 x 1x128 GEMM
    equals the fp64 product of the dequantized operands, blocked down the tokens."""
    M, N, K = 256, 384, 256          # tokens, output features, input features
    dy = synth.activations(M, N, seed=11, sub=synth.SUB_DY)
    x = synth.activations(M, K, seed=11, sub=synth.SUB_X)
    dyq, dys = orc.quant_act_1x128_t(dy, mode)        # [N, M], [N, M/128]
    xq, xs = orc.quant_act_1x128_t(x, mode)           # [K, M], [K, M/128]
    assert dyq.shape == (N, M) and dys.shape == (N, M // 128) and xq.shape == (K, M)
    dw = orc.gemm_1x128(dyq, dys, xq, xs)
    ref = _dequant_row_scaled(orc, dyq, dys) @ _dequant_row_scaled(orc, xq, xs).T
    rms = np.sqrt(np.mean(ref ** 2))
    assert dw.shape == (N, K) and rms > 0
    assert np.max(np.abs(dw - ref)) <= 1e-12 * rms * np.sqrt(M)
    # a block of the transposed quantization is a column block of X: its scale is the
    # column's amax over 128 tokens
    col = synth.bf16_bits_to_f32(x[:128, 5]).astype(np.float64)
    assert xs[5, 0] == np.float32(orc.block_scale(float(np.max(np.abs(col))), mode))
    # sampled positions agree with the full product
    rows, cols = np.array([0, 17, 383, 200]), np.array([255, 0, 128, 77])
    assert np.array_equal(orc.gemm_1x128_sampled(dyq, dys, xq, xs, rows, cols), dw[rows, cols])


def test_gemm_1x128_reduces_to_block_scaled_gemm(orc):
    """Row scales that are constant over each 128-row group are 128x128 block scales:
    the two GEMMs then agree exactly."""
    M, N, K = 130, 256, 384
    xq, xs, wq, ws = _operands(orc, M, N, K, seed=3)
    ws_rows = np.repeat(ws, 128, axis=0)               # [N, K/128]
    assert np.array_equal(orc.gemm_1x128(xq, xs, wq, ws_rows), orc.gemm(xq, xs, wq, ws))


def test_gemm_integer_special_case(orc):
    """All scales 1 and codes of small integers: Y is an exact integer matmul."""
    g = np.random.default_rng(5)
    # codes of the integers 0..8 and their negatives: 0x00 0x38 0x40 0x44 0x48 0x4A 0x4C 0x4E 0x50
    int_codes = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], dtype=np.uint8)
    M, N, K = 64, 128, 384
    ix = g.integers(0, 9, (M, K))
    iw = g.integers(0, 9, (N, K))
    sx = g.integers(0, 2, (M, K))
    sw = g.integers(0, 2, (N, K))
    xq = int_codes[ix] | (sx * 0x80).astype(np.uint8)
    wq = int_codes[iw] | (sw * 0x80).astype(np.uint8)
    vx = ix * (1 - 2 * sx)
    vw = iw * (1 - 2 * sw)
    y = orc.gemm(xq, np.ones((M, K // 128), np.float32), wq, np.ones((N // 128, K // 128), np.float32))
    assert np.array_equal(y, (vx @ vw.T).astype(np.float64))


def test_gemm_single_block_is_scaled_dot(orc):
    """K = 128: Y = xs * ws * P with P the exact dot product of the decoded codes."""
    xq, xs, wq, ws = _operands(orc, 16, 256, 128, seed=3)
    y = orc.gemm(xq, xs, wq, ws)
    P = orc.e4m3_decode_array(xq) @ orc.e4m3_decode_array(wq).T  # exact: 2^-18 grid, < 2^43
    ref = (xs.astype(np.float64) @ np.ones((1, 256))) * np.repeat(ws[:, 0].astype(np.float64), 128)[None, :] * P
    assert np.array_equal(y, ref)


def test_gemm_sampled_equals_full(orc):
    xq, xs, wq, ws = _operands(orc, 96, 256, 384, seed=4)
    y = orc.gemm(xq, xs, wq, ws)
    g = np.random.default_rng(1)
    rows = g.integers(0, 96, 500)
    cols = g.integers(0, 256, 500)
    assert np.array_equal(orc.gemm_sampled(xq, xs, wq, ws, rows, cols), y[rows, cols])


def _grouped_operands(orc, counts, N, K, seed, mode=0):
    offs = synth.offsets_from_counts(counts)
    M = int(offs[-1])
    E = len(counts)
    x = synth.activations(max(M, 1), K, seed=seed)[:M]
    w = synth.expert_weights(E, N, K, seed=seed)
    xq, xs = orc.quant_act_1x128(x, mode)
    wq = np.empty((E, N, K), np.uint8)
    ws = np.empty((E, N // 128, K // 128), np.float32)
    for e in range(E):
        wq[e], ws[e] = orc.quant_w_128x128(w[e], mode)
    return xq, xs, wq, ws, offs


@pytest.mark.parametrize("counts", [[5, 0, 129, 1, 64], [0, 0, 3], [128, 128], [0]])
def test_grouped_equals_per_expert_gemms(orc, counts):
    N, K = 256, 384
    xq, xs, wq, ws, offs = _grouped_operands(orc, counts, N, K, seed=len(counts))
    y = orc.grouped_gemm(xq, xs, wq, ws, offs)
    assert y.shape == (sum(counts), N)
    for e in range(len(counts)):
        a, b = offs[e], offs[e + 1]
        if b > a:
            ref = _dequant_rows(orc, xq[a:b], xs[a:b]) @ _dequant_tiles(orc, wq[e], ws[e]).T
            rms = np.sqrt(np.mean(ref ** 2))
            assert np.max(np.abs(y[a:b] - ref)) <= 1e-12 * rms * np.sqrt(K)
            assert np.array_equal(y[a:b], orc.gemm(xq[a:b], xs[a:b], wq[e], ws[e]))
    if y.size:
        g = np.random.default_rng(2)
        rows = g.integers(0, y.shape[0], 200)
        cols = g.integers(0, N, 200)
        assert np.array_equal(orc.grouped_gemm_sampled(xq, xs, wq, ws, offs, rows, cols), y[rows, cols])


def test_routing_counts():
    row_token, offs = synth.moe_routing(8192, 128, 8, seed=0)
    assert offs[0] == 0 and offs[-1] == 65536 and row_token.size == 65536
    counts = np.diff(offs)
    assert (counts >= 0).all()
    # each token appears exactly top-k times
    assert (np.bincount(row_token, minlength=8192) == 8).all()
    # rows are ordered by token inside each expert group
    for e in range(0, 128, 17):
        seg = row_token[offs[e]:offs[e + 1]]
        assert (np.diff(seg) > 0).all()


# ---- the full-output GEMMs (codes decoded once, block sums in fp64) ---------------

def test_full_gemm_table_is_decode_times_512(orc):
    """Every entry of the full-output GEMMs' table is decode(c) * 2^9: an integer of
    magnitude <= 229376 for the 254 finite codes, NaN for 0x7F and 0xFF."""
    t = orc.e4m3_x512_table()
    for c in range(256):
        d = orc.e4m3_decode(c)
        if c in (0x7F, 0xFF):
            assert np.isnan(t[c]) and np.isnan(d)
        else:
            assert t[c] == d * 512.0 and t[c] == np.round(t[c]) and abs(t[c]) <= 229376
    assert t[0x7E] == 448 * 512 and t[0x01] == 1 and t[0x38] == 512 and t[0x80] == 0


@pytest.mark.parametrize("shape", [(256, 512, 512), (1, 128, 128), (17, 256, 384), (130, 384, 1024), (9, 128, 2048)])
@pytest.mark.parametrize("mode", [0, 1])
def test_full_gemm_bit_identical_to_elementwise(orc, shape, mode):
    """gemm_full computes the same fp64 numbers as gemm, bit for bit (each block sum
    is exact in both; the scale products and the ascending sum over blocks are the
    same operations)."""
    M, N, K = shape
    xq, xs, wq, ws = _operands(orc, M, N, K, seed=M * 3 + K, mode=mode)
    a = orc.gemm(xq, xs, wq, ws)
    b = orc.gemm_full(xq, xs, wq, ws)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))
    # and the closed form holds for it directly
    ref = _dequant_rows(orc, xq, xs) @ _dequant_tiles(orc, wq, ws).T
    assert np.max(np.abs(b - ref)) <= 1e-12 * np.sqrt(np.mean(ref ** 2)) * np.sqrt(K)


def test_full_gemm_extreme_codes_exact(orc):
    """Blocks of +-448 codes (the largest products, 128 * 448^2 per block) and of the
    smallest subnormal: the fp64 block sums stay exact, so unit scales give the exact
    integer result."""
    M, N, K = 4, 128, 256
    xq = np.full((M, K), 0x7E, np.uint8)
    xq[1] = 0xFE
    xq[2] = 0x01
    xq[3, :128] = 0x7E
    xq[3, 128:] = 0x81
    wq = np.full((N, K), 0x7E, np.uint8)
    wq[::2] = 0x01
    xs = np.ones((M, K // 128), np.float32)
    ws = np.ones((N // 128, K // 128), np.float32)
    y = orc.gemm_full(xq, xs, wq, ws)
    big, tiny = 448.0, 2.0 ** -9
    assert y[0, 1] == K * big * big and y[1, 1] == -K * big * big
    assert y[0, 0] == K * big * tiny and y[2, 0] == K * tiny * tiny
    assert y[3, 1] == 128 * big * big - 128 * tiny * big
    assert np.array_equal(y.view(np.uint64), orc.gemm(xq, xs, wq, ws).view(np.uint64))


def test_full_gemm_1x128_bit_identical(orc):
    M, N, K = 70, 256, 384
    g = np.random.default_rng(11)
    xq = g.integers(0, 256, (M, K), dtype=np.uint8)
    wq = g.integers(0, 256, (N, K), dtype=np.uint8)
    xq[xq & 0x7F == 0x7F] = 0x10
    wq[wq & 0x7F == 0x7F] = 0x10
    xs = g.uniform(0.5, 2, (M, K // 128)).astype(np.float32)
    ws = g.uniform(0.5, 2, (N, K // 128)).astype(np.float32)
    a = orc.gemm_1x128(xq, xs, wq, ws)
    b = orc.gemm_1x128_full(xq, xs, wq, ws)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


@pytest.mark.parametrize("offs", [[0, 5, 5, 134, 135, 199, 300], [0, 0, 0, 7], [0, 128, 256, 512],
                                  [0, 10, 3, 20, 40], [0, 10, 20, 15, 40]],
                         ids=["ragged", "leading_empty", "aligned", "malformed_dip", "malformed_overlap"])
def test_full_grouped_bit_identical(orc, offs):
    """grouped_gemm_full matches grouped_gemm bit for bit, including which expert
    owns each row when the offsets are not monotone, and NaN rows that no expert owns."""
    E, N, K = len(offs) - 1, 256, 384
    M = max(offs)
    offs = np.array(offs, np.int32)
    x = synth.activations(M, K, seed=3)
    w = synth.expert_weights(E, N, K, seed=3, sub=synth.SUB_W)
    xq, xs = orc.quant_act_1x128(x)
    wq, ws = orc.quant_w_128x128(w.reshape(E * N, K))
    wq, ws = wq.reshape(E, N, K), ws.reshape(E, N // 128, K // 128)
    a = orc.grouped_gemm(xq, xs, wq, ws, offs)
    b = orc.grouped_gemm_full(xq, xs, wq, ws, offs)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok].view(np.uint64), b[ok].view(np.uint64))
