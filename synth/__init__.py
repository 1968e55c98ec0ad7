"""Seeded synthetic inputs for the block-FP8 linear layer.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It draws random numbers and lays them out in the shapes of the
workloads; it holds none of the quantization or GEMM arithmetic, and it imports
neither the oracle nor the GPU library.

Workload recipe (the article "NVIDIA NeMo RL achieves 48% speedup with
end-to-end FP8 precision training", Jessie A Ellis, Apr 20 2026, names the
model families -- Llama 3.1 8B, Qwen3-30B MoE -- but prints no tensors, so all
values are synthetic):

* activations: fp32 N(0, 1); each entry independently, with probability 1e-3,
  is multiplied by 50 (outliers); then rounded to bf16 (round to nearest even);
* weights: fp32 0.02 * N(0, 1), rounded to bf16;
* output gradients dY (training backward): the activation recipe, from
  their own sub-stream (the article prints no gradient statistics; block
  scaling makes every result invariant to a common power-of-2 factor);
* gate+up projection outputs (the gated activation's input, [M, 2F], gate
  columns first): the activation recipe scaled by 2, about the spread of an
  8B-shaped gate+up GEMM over the inputs above (0.02 * sqrt(4096) = 1.28
  per unit input, inputs of rms about 1.9 with the outliers); the outliers
  reach |g| of several hundred, so both tails of the logistic function are
  exercised;
* MoE router: fp32 N(0, 1) logits [tokens, experts]; each token goes to its
  top-k experts by logit (softmax is monotone, so this is top-k by
  probability), ties to the lower expert id; rows are grouped by expert, then
  ordered by token, and the group offsets are the prefix sums of the counts.

Every generator is keyed by (seed, sub-stream) through numpy's PCG64, so the
same bytes reach the GPU and the oracle.  The ``*_dev`` generators draw the
same recipes directly on a device with torch's seeded device generator: they
serve the benchmark's large timing inputs, whose bytes no oracle compares.
"""

from __future__ import annotations

import numpy as np
import torch

SEED = 0
SUB_X = 0
SUB_W = 1
SUB_ROUTER = 2
SUB_DY = 3      # output gradients of the backward (data-gradient) product
SUB_GU = 4      # gate+up projection outputs (the gated activation's input)


def sub_layer(layer: int) -> int:
    """Sub-stream id of the weights of transformer layer ``layer``."""
    return 100 + int(layer)


def _rng(seed: int, sub: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(sub)])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest even) and return the raw 16-bit payloads."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen raw bf16 payloads to fp32 (exact: bf16 is the top half of fp32)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(M: int, K: int, seed: int = SEED, sub: int = SUB_X,
                outlier_p: float = 1e-3, outlier_mul: float = 50.0) -> np.ndarray:
    """bf16 payloads [M, K]: N(0,1) with Bernoulli(outlier_p) entries x outlier_mul."""
    g = _rng(seed, sub)
    x = g.standard_normal((M, K), dtype=np.float32)
    mask = g.random((M, K), dtype=np.float32) < np.float32(outlier_p)
    x[mask] *= np.float32(outlier_mul)
    return f32_to_bf16_bits(x)


def gate_up(M: int, F: int, seed: int = SEED, sub: int = SUB_GU, std: float = 2.0) -> np.ndarray:
    """bf16 payloads [M, 2F]: gate columns 0..F-1, up columns F..2F-1; the
    activation recipe (N(0,1), Bernoulli(1e-3) entries x 50) times ``std``."""
    g = _rng(seed, sub)
    x = g.standard_normal((M, 2 * F), dtype=np.float32)
    mask = g.random((M, 2 * F), dtype=np.float32) < np.float32(1e-3)
    x[mask] *= np.float32(50.0)
    return f32_to_bf16_bits(x * np.float32(std))


def weights(N: int, K: int, seed: int = SEED, sub: int = SUB_W, std: float = 0.02) -> np.ndarray:
    """bf16 payloads [N, K]: std * N(0, 1)."""
    g = _rng(seed, sub)
    w = g.standard_normal((N, K), dtype=np.float32)
    w *= np.float32(std)
    return f32_to_bf16_bits(w)


def expert_weights(E: int, N: int, K: int, seed: int = SEED, sub: int = SUB_W,
                   std: float = 0.02) -> np.ndarray:
    """bf16 payloads [E, N, K]: std * N(0, 1), one draw for all experts."""
    g = _rng(seed, sub)
    w = g.standard_normal((E, N, K), dtype=np.float32)
    w *= np.float32(std)
    return f32_to_bf16_bits(w)


def _dev_gen(seed: int, sub: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) * 1000003 + int(sub))
    return g


def activations_dev(M: int, K: int, device, seed: int = SEED, sub: int = SUB_X,
                    outlier_p: float = 1e-3, outlier_mul: float = 50.0) -> torch.Tensor:
    """bf16 tensor [M, K] on ``device``: the activation recipe, drawn on the device."""
    g = _dev_gen(seed, sub, device)
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    hit = torch.rand((M, K), generator=g, device=device, dtype=torch.float32) < outlier_p
    x = torch.where(hit, x * outlier_mul, x)
    return x.to(torch.bfloat16)


def weights_dev(N: int, K: int, device, seed: int = SEED, sub: int = SUB_W, std: float = 0.02) -> torch.Tensor:
    """bf16 tensor [N, K] on ``device``: std * N(0, 1), drawn on the device."""
    g = _dev_gen(seed, sub, device)
    return (torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std).to(torch.bfloat16)


def moe_routing(tokens: int, experts: int, topk: int, seed: int = SEED,
                sub: int = SUB_ROUTER):
    """Top-k routing of N(0,1) logits.

    Returns ``(row_token, offsets)``: ``row_token[r]`` is the token whose
    activation row ``r`` of the expert-grouped matrix holds, and ``offsets``
    (int32, length experts + 1) are the prefix sums of the per-expert counts.
    """
    g = _rng(seed, sub)
    logits = g.standard_normal((tokens, experts), dtype=np.float32)
    # stable sort of the negated logits: equal logits keep the lower expert id first
    choice = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    exp = choice.reshape(-1).astype(np.int64)
    order = np.lexsort((tok, exp))
    row_token = tok[order]
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return row_token, offsets


def moe_dest(row_token, tokens: int, topk: int) -> np.ndarray:
    """The routing seen from the tokens: int32 [tokens, topk], entry (t, k) the row of the
    expert-grouped matrix that holds token t's k-th copy (in row order), -1 where token t
    has fewer than topk copies.  The inverse of ``row_token``."""
    rt = np.asarray(row_token, dtype=np.int64)
    dest = np.full((tokens, topk), -1, dtype=np.int32)
    seen = np.zeros(tokens, dtype=np.int64)
    for m, t in enumerate(rt):
        dest[t, seen[t]] = m
        seen[t] += 1
    return dest


def offsets_from_counts(counts) -> np.ndarray:
    """int32 group offsets (length E + 1) for explicit per-expert row counts."""
    c = np.asarray(counts, dtype=np.int64)
    out = np.zeros(c.size + 1, dtype=np.int32)
    out[1:] = np.cumsum(c)
    return out


# ---------------------------------------------------------------------------
# Enumeration of (x, amax) bf16 pairs laid out as 1x128 blocks.
#
# The code of an element depends only on its own value x and on the block's
# amax, so covering every bf16 pair with |x| <= amax covers every decision the
# activation quantizer can take.  Each block holds amax in slot 0 and up to 127
# values x in slots 1..127 (unused slots hold +0).  ``sign`` flips every value
# of the block (negative x, amax element included).
# ---------------------------------------------------------------------------

BF16_MAX_FINITE_BITS = 0x7F7F


def pair_blocks(amax_lo: int, amax_hi: int, sign: int = 0) -> np.ndarray:
    """bf16 payloads [nblocks, 128] for every amax payload in [amax_lo, amax_hi)
    and every x payload in [0, amax]."""
    a = np.arange(int(amax_lo), int(amax_hi), dtype=np.int32)
    nx = a + 1
    nblk = (nx + 126) // 127
    blk_a = np.repeat(a, nblk)
    first = np.repeat(np.cumsum(nblk) - nblk, nblk).astype(np.int32)
    j = np.arange(blk_a.size, dtype=np.int32) - first
    x = (j * 127)[:, None] + np.arange(127, dtype=np.int32)[None, :]
    x[x > blk_a[:, None]] = 0
    out = np.empty((blk_a.size, 128), dtype=np.uint16)
    out[:, 0] = blk_a
    out[:, 1:] = x
    if sign:
        out |= np.uint16(0x8000)
    return out


def pair_block_ranges(max_elems: int = 1 << 26):
    """Split [1, BF16_MAX_FINITE_BITS] into amax ranges whose pair blocks hold
    at most about ``max_elems`` elements each."""
    ranges = []
    lo = 1
    acc = 0
    for a in range(1, BF16_MAX_FINITE_BITS + 1):
        acc += ((a + 1 + 126) // 127) * 128
        if acc >= max_elems:
            ranges.append((lo, a + 1))
            lo = a + 1
            acc = 0
    if lo <= BF16_MAX_FINITE_BITS:
        ranges.append((lo, BF16_MAX_FINITE_BITS + 1))
    return ranges
