// fp8bs_quant.hip -- 1x128 activation and 128x128 weight quantizers (gfx950).
//
// The article "NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
// precision training", section "Technical breakthrough", quantizes
// activations per 1x128 block and weights per 128x128 block to E4M3; section
// "Real-world performance gains" re-quantizes the weights after every
// training step.  Both kernels move each byte once (read bf16, write codes and
// one fp32 per block) and are bound by HBM bandwidth; the per-element work is
// kept to a handful of VALU operations so that they stay there:
//   amax      : packed 16-bit integer max over magnitude payloads, then a
//               16-lane DPP butterfly (activations) or a workgroup reduction
//               (weights);
//   quotient  : EXACT mode runs the 5-operation Newton division of
//               fp8bs_device.hpp (bit-exact with IEEE division), POW2 mode a
//               single exact multiply by 2^-k;
//   encoding  : v_cvt_pk_fp8_f32, two codes per instruction.
#include "fp8bs_device.hpp"
#include "fp8bs_internal.hpp"

namespace fp8bs {

// ---- activations: 1x128 blocks ------------------------------------------------
//
// A row-major [M, K] tensor with K % 128 == 0 is a flat sequence of
// M*K/128 blocks of 256 contiguous bytes, and xs[m, kb] is entry m*K/128+kb
// of the same sequence, so the kernel works on block indices only.  Each
// 16-lane DPP row of a wave owns one block per step (16 lanes x 16 bytes);
// a wave's four rows cover 4 consecutive blocks, i.e. 1 KiB of contiguous
// bf16 per load instruction, and each lane keeps QA_UNROLL loads in flight.
// Two (8 blocks per wave) measured best on gfx950: against four and eight,
// more, shorter waves fill the chip sooner at the sizes of a layer's
// activations (8192 x 4096: 19.5 us against 21.1 with four); one load per lane
// leaves too little in flight on the large shapes.
constexpr int QA_UNROLL = 2;
constexpr int QA_THREADS = 256;
constexpr int QA_BLOCKS_PER_WG = (QA_THREADS / 64) * 4 * QA_UNROLL;

template <int MODE>
__global__ __launch_bounds__(QA_THREADS) void quant_act_kernel(const u32x4 *__restrict__ x, u32x2 *__restrict__ q,
                                                               float *__restrict__ s, int64_t nblocks)
{
    const int lane = threadIdx.x & 63;
    const int slot = lane >> 4; // block slot of this DPP row
    const int c = lane & 15;    // 16-byte chunk within the block
    const int64_t wave = (int64_t)blockIdx.x * (QA_THREADS / 64) + (threadIdx.x >> 6);
    const int64_t b0 = wave * (4 * QA_UNROLL) + slot;

    u32x4 v[QA_UNROLL];
#pragma unroll
    for (int j = 0; j < QA_UNROLL; ++j) {
        const int64_t b = b0 + 4 * j;
        v[j] = (b < nblocks) ? __builtin_nontemporal_load(x + b * 16 + c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < QA_UNROLL; ++j) {
        const int64_t b = b0 + 4 * j;
        // every lane takes part in the DPP reduction (blocks past the end hold zeros)
        const float amax = amax_value(row16_max(chunk_max_mag(v[j])));
        BlockQuant<MODE> bq;
        bq.init(amax);
        const u32x2 codes = quant_chunk<MODE>(v[j], bq);
        if (b < nblocks) {
            __builtin_nontemporal_store(codes, q + b * 16 + c);
            if (c == 0)
                s[b] = bq.s;
        }
    }
}

hipError_t launch_quant_act(const void *x, int64_t M, int64_t K, void *xq, float *xs, int mode, hipStream_t stream)
{
    const int64_t nblocks = M * (K / 128);
    if (nblocks == 0)
        return hipSuccess;
    const int64_t grid = (nblocks + QA_BLOCKS_PER_WG - 1) / QA_BLOCKS_PER_WG;
    if (mode == SCALE_POW2)
        return launch(quant_act_kernel<SCALE_POW2>, dim3((unsigned)grid), dim3(QA_THREADS), 0, stream,
                      (const u32x4 *)x, (u32x2 *)xq, xs, nblocks);
    return launch(quant_act_kernel<SCALE_EXACT>, dim3((unsigned)grid), dim3(QA_THREADS), 0, stream,
                  (const u32x4 *)x, (u32x2 *)xq, xs, nblocks);
}

// ---- weights: 128x128 blocks -----------------------------------------------------
//
// One 256-thread workgroup per 128x128 block.  Thread t covers the 16-byte
// chunk (t % 16) of rows t/16, t/16 + 16, ..., t/16 + 112: eight loads in
// flight per thread, the whole 32 KiB block held in registers across the
// amax reduction, so the bf16 input is read from HBM exactly once.
// A launch covers up to QW_MAX_TENSORS tensors; workgroup ids are
// concatenated over the tensors' block grids.
constexpr int QW_THREADS = 256;
constexpr int QW_MAX_TENSORS = 32;

struct QWArgs {
    int count;
    int64_t tile_begin[QW_MAX_TENSORS + 1];
    const uint16_t *w[QW_MAX_TENSORS];
    uint8_t *q[QW_MAX_TENSORS];
    float *s[QW_MAX_TENSORS];
    int64_t K[QW_MAX_TENSORS];
};

template <int MODE>
__global__ __launch_bounds__(QW_THREADS) void quant_w_kernel(QWArgs a)
{
    __shared__ uint32_t red[QW_THREADS / 64];
    const int64_t tile = blockIdx.x;
    int i = 0;
    while (i + 1 < a.count && tile >= a.tile_begin[i + 1])
        ++i;
    const int64_t K = a.K[i];
    const int64_t KB = K / 128;
    const int64_t local = tile - a.tile_begin[i];
    const int64_t nb = local / KB, kb = local % KB;

    const int t = threadIdx.x;
    const int r0 = t >> 4, c = t & 15;
    const int64_t base = (nb * 128 + r0) * K + kb * 128 + c * 8; // element offset of this thread's first chunk
    const int64_t rstep = 16 * K;                                // 16 rows
    const uint16_t *w = a.w[i];

    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = __builtin_nontemporal_load((const u32x4 *)(w + base + j * rstep));

    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t cm = chunk_max_mag(v[j]);
        m = m > cm ? m : cm;
    }
    m = row16_max(m);
    {
        const uint32_t a0 = __builtin_amdgcn_readlane(m, 0), a1 = __builtin_amdgcn_readlane(m, 16);
        const uint32_t a2 = __builtin_amdgcn_readlane(m, 32), a3 = __builtin_amdgcn_readlane(m, 48);
        uint32_t wm = a0 > a1 ? a0 : a1;
        const uint32_t wm2 = a2 > a3 ? a2 : a3;
        wm = wm > wm2 ? wm : wm2;
        if ((t & 63) == 0)
            red[t >> 6] = wm;
    }
    __syncthreads();
    uint32_t bm = red[0];
#pragma unroll
    for (int j = 1; j < QW_THREADS / 64; ++j)
        bm = bm > red[j] ? bm : red[j];

    BlockQuant<MODE> bq;
    bq.init(amax_value(bm));
    uint8_t *q = a.q[i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x2 codes = quant_chunk<MODE>(v[j], bq);
        __builtin_nontemporal_store(codes, (u32x2 *)(q + base + j * rstep));
    }
    if (t == 0)
        a.s[i][nb * KB + kb] = bq.s;
}

hipError_t launch_quant_w(const WTensor *t, int64_t count, int mode, hipStream_t stream)
{
    for (int64_t first = 0; first < count; first += QW_MAX_TENSORS) {
        QWArgs a = {};
        const int64_t n = (count - first) < QW_MAX_TENSORS ? (count - first) : QW_MAX_TENSORS;
        int64_t tiles = 0;
        for (int64_t j = 0; j < n; ++j) {
            const WTensor &wt = t[first + j];
            a.tile_begin[j] = tiles;
            a.w[j] = (const uint16_t *)wt.w;
            a.q[j] = (uint8_t *)wt.q;
            a.s[j] = wt.s;
            a.K[j] = wt.K;
            tiles += (wt.N / 128) * (wt.K / 128);
        }
        a.tile_begin[n] = tiles;
        a.count = (int)n;
        if (tiles == 0)
            continue;
        hipError_t e = (mode == SCALE_POW2)
                           ? launch(quant_w_kernel<SCALE_POW2>, dim3((unsigned)tiles), dim3(QW_THREADS), 0, stream, a)
                           : launch(quant_w_kernel<SCALE_EXACT>, dim3((unsigned)tiles), dim3(QW_THREADS), 0, stream, a);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

} // namespace fp8bs
