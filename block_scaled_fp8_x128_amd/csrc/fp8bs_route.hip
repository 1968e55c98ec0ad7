// fp8bs_route.hip -- MoE dispatch: the 1x128 activation quantizer reading its
// rows through an index.
//
// The article "NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
// precision training" runs its recipe on a mixture-of-experts model
// (Qwen3-30B, section "Real-world performance gains") with activations
// quantized per 1x128 block (section "Technical breakthrough").  An MoE layer
// sends every token to several experts, so the grouped GEMM's input holds
// each token's row once per expert, in expert order.  The 1x128 blocks lie
// along a row, so quantizing the gathered rows gives the same codes and scales
// as gathering the quantized rows; this kernel does the gather and the
// quantization in one pass:
//
//   xq[m, :], xs[m, :] = quant_act_1x128(x[rows[m], :])
//
// reading each token's bf16 row from the [T, K] token tensor (a few tens of
// MB, which stays in the caches across its repeats) instead of a
// materialized [M, K] copy.  Block layout and encoder are the activation
// quantizer's: each 16-lane DPP row owns one 1x128 block, 16 bytes per lane.
// An index outside [0, T) reads as an all-zero row (codes 0, scale 1); no
// address outside x is formed.
#include "fp8bs_device.hpp"
#include "fp8bs_internal.hpp"

namespace fp8bs {

constexpr int RG_UNROLL = 2;
constexpr int RG_THREADS = 256;
constexpr int RG_BLOCKS_PER_WG = (RG_THREADS / 64) * 4 * RG_UNROLL;

template <int MODE>
__global__ __launch_bounds__(RG_THREADS) void quant_act_gather_kernel(const uint16_t *__restrict__ x, int64_t T,
                                                                    const int32_t *__restrict__ rows,
                                                                    u32x2 *__restrict__ q, float *__restrict__ s,
                                                                    uint32_t nblocks, uint32_t KB)
{
    const int lane = threadIdx.x & 63;
    const int slot = lane >> 4; // block slot of this DPP row
    const int c = lane & 15;    // 16-byte chunk within the block
    const uint32_t wave = blockIdx.x * (RG_THREADS / 64) + (threadIdx.x >> 6);
    const uint32_t b0 = wave * (4 * RG_UNROLL) + slot;
    const int64_t K = (int64_t)KB * 128;

    u32x4 v[RG_UNROLL];
#pragma unroll
    for (int j = 0; j < RG_UNROLL; ++j) {
        const uint32_t b = b0 + 4 * j;
        v[j] = u32x4{0u, 0u, 0u, 0u};
        if (b < nblocks) {
            const uint32_t m = b / KB, kb = b - m * KB;
            const int64_t r = rows[m];
            // an ordinary (cached) load: each token row is read once per expert it
            // is routed to, and the token tensor fits the caches, so its repeats
            // hit there (a nontemporal load sent every repeat to HBM)
            if (r >= 0 && r < T)
                v[j] = *((const u32x4 *)(x + r * K + (int64_t)kb * 128) + c);
        }
    }
#pragma unroll
    for (int j = 0; j < RG_UNROLL; ++j) {
        const uint32_t b = b0 + 4 * j;
        // every lane takes part in the DPP reduction (blocks past the end hold zeros)
        const float amax = amax_value(row16_max(chunk_max_mag(v[j])));
        BlockQuant<MODE> bq;
        bq.init(amax);
        const u32x2 codes = quant_chunk<MODE>(v[j], bq);
        if (b < nblocks) {
            __builtin_nontemporal_store(codes, q + (int64_t)b * 16 + c);
            if (c == 0)
                s[b] = bq.s;
        }
    }
}

hipError_t launch_quant_act_gather(const void *x, int64_t T, int64_t K, const int32_t *rows, int64_t M, void *xq,
                                   float *xs, int mode, hipStream_t stream)
{
    const int64_t nblocks = M * (K / 128);
    if (nblocks == 0)
        return hipSuccess;
    const int64_t grid = (nblocks + RG_BLOCKS_PER_WG - 1) / RG_BLOCKS_PER_WG;
    if (mode == SCALE_POW2)
        return launch(quant_act_gather_kernel<SCALE_POW2>, dim3((unsigned)grid), dim3(RG_THREADS), 0, stream,
                      (const uint16_t *)x, T, rows, (u32x2 *)xq, xs, (uint32_t)nblocks, (uint32_t)(K / 128));
    return launch(quant_act_gather_kernel<SCALE_EXACT>, dim3((unsigned)grid), dim3(RG_THREADS), 0, stream,
                  (const uint16_t *)x, T, rows, (u32x2 *)xq, xs, (uint32_t)nblocks, (uint32_t)(K / 128));
}

// The same dispatch from the token side: each token row is read once and
// quantized once, and its codes and scales go to every destination row the
// routing gives it:
//
//   for t < T, k < topk, d = dest[t * topk + k] in [0, M):  xq[d, :], xs[d, :] = quant_act_1x128(x[t, :])
//
// Reading each token once (instead of once per expert) leaves the codes'
// writes as the main traffic.  Blocks are those of quant_act_1x128 over x
// (one 16-lane DPP row per 1x128 block); the destinations of a block's token
// are uniform over its DPP row, so every store is one block's 128 contiguous
// code bytes.  Destinations outside [0, M) are skipped; rows no entry names
// are not written.
template <int MODE>
__global__ __launch_bounds__(RG_THREADS) void quant_act_scatter_kernel(const uint16_t *__restrict__ x,
                                                                     const int32_t *__restrict__ dest, int topk,
                                                                     int64_t M, u32x2 *__restrict__ q,
                                                                     float *__restrict__ s, uint32_t nblocks,
                                                                     uint32_t KB)
{
    const int lane = threadIdx.x & 63;
    const int slot = lane >> 4;
    const int c = lane & 15;
    const uint32_t wave = blockIdx.x * (RG_THREADS / 64) + (threadIdx.x >> 6);
    const uint32_t b0 = wave * (4 * RG_UNROLL) + slot;

    u32x4 v[RG_UNROLL];
#pragma unroll
    for (int j = 0; j < RG_UNROLL; ++j) {
        const uint32_t b = b0 + 4 * j;
        v[j] = (b < nblocks) ? __builtin_nontemporal_load((const u32x4 *)x + (int64_t)b * 16 + c)
                             : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < RG_UNROLL; ++j) {
        const uint32_t b = b0 + 4 * j;
        // every lane takes part in the DPP reduction (blocks past the end hold zeros)
        const float amax = amax_value(row16_max(chunk_max_mag(v[j])));
        BlockQuant<MODE> bq;
        bq.init(amax);
        const u32x2 codes = quant_chunk<MODE>(v[j], bq);
        if (b < nblocks) {
            const uint32_t t = b / KB, kb = b - t * KB;
            const int32_t *dt = dest + (int64_t)t * topk;
            for (int k = 0; k < topk; ++k) {
                const int64_t d = dt[k];
                if (d >= 0 && d < M) {
                    __builtin_nontemporal_store(codes, q + (d * KB + kb) * 16 + c);
                    if (c == 0)
                        s[d * KB + kb] = bq.s;
                }
            }
        }
    }
}

hipError_t launch_quant_act_scatter(const void *x, int64_t T, int64_t K, const int32_t *dest, int64_t topk,
                                    int64_t M, void *xq, float *xs, int mode, hipStream_t stream)
{
    const int64_t nblocks = T * (K / 128);
    if (nblocks == 0 || topk == 0)
        return hipSuccess;
    const int64_t grid = (nblocks + RG_BLOCKS_PER_WG - 1) / RG_BLOCKS_PER_WG;
    if (mode == SCALE_POW2)
        return launch(quant_act_scatter_kernel<SCALE_POW2>, dim3((unsigned)grid), dim3(RG_THREADS), 0, stream,
                      (const uint16_t *)x, dest, (int)topk, M, (u32x2 *)xq, xs, (uint32_t)nblocks,
                      (uint32_t)(K / 128));
    return launch(quant_act_scatter_kernel<SCALE_EXACT>, dim3((unsigned)grid), dim3(RG_THREADS), 0, stream,
                  (const uint16_t *)x, dest, (int)topk, M, (u32x2 *)xq, xs, (uint32_t)nblocks, (uint32_t)(K / 128));
}

} // namespace fp8bs
