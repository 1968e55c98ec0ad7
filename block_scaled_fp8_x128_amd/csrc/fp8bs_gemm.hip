// fp8bs_gemm.hip -- block-scaled FP8 GEMM and its grouped (MoE) form, gfx950.
//
// The article "NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
// precision training", section "Technical breakthrough": linear layers run FP8
// math on operands quantized per 1x128 (activations) and 128x128 (weights)
// block.  Here
//   Y[m, n] = sum_kb (xs[m, kb] * ws[n/128, kb]) * P[m, n, kb],
//   P[m, n, kb] = sum_{k in kb} decode(xq[m, k]) * decode(wq[n, k]),
// with P from the CDNA4 FP8 matrix cores into a fresh fp32 partial per
// 128-wide K block, and the fp32 scale product applied by one FMA per output
// element and K block into the running fp32 accumulator.  The MFMA builtin
// is the block-scaled one; with its scale operands 0 the compiler emits the
// plain v_mfma_f32_16x16x128_f8f6f4, whose products equal those of the
// scaled form with E8M0 127 = 2^0 bit for bit, without holding the neutral
// scale in a VGPR (1-3% faster on the 8B-shaped GEMMs).
//
// Tiling.  A workgroup computes a BM x BN tile of Y with WAVES_M x WAVES_N
// waves, each wave a (BM/WAVES_M) x (BN/WAVES_N) sub-tile made of 16x16
// MFMA tiles.  One MFMA consumes a whole 128-wide K block (one scale pair),
// so the K loop steps one scale block at a time.  Both operands are
// K-contiguous (Y = X W^T), so A- and B-fragments load the same way: lane l
// takes row l % 16 and the 32-byte K slice (l / 16); the MFMA's A operand is
// the weight tile and its B operand the activation tile, which leaves each
// lane holding 4 consecutive n of one m -- one 16-byte (fp32) or 8-byte
// (bf16) store per MFMA tile.
//
// Kernels in this file:
//   gemm_dma_kernel       the persistent large-tile GEMM (256x256 or 128x256
//                         tiles, operands loaded straight into LDS), also split
//                         along K for few-tile products, grouped over experts,
//                         and with power-of-2 scales applied by the matrix core;
//   splitk_reduce_kernel  adds the K ranges of a split product;
//   grouped_tile_table_kernel  the row tiles of a grouped launch;
//   gemm_skinny_kernel    weight streaming for at most 16 activation rows;
//   gemm_kernel           the general 128x128 GEMM (N not a multiple of 256):
//                         global -> registers -> LDS, double-buffered, one
//                         barrier per K block; LDS rows are 128 bytes and the
//                         16-byte chunk c of row r sits at chunk c ^ ((r >> 1)
//                         & 7), so the 16 rows one 16-lane group reads spread
//                         over all banks.
// The launchers at the end pick one per shape (the variant table).
//
// Workgroup order.  Consecutive workgroup ids are dispatched round-robin to
// the 8 XCDs, each with its own L2; ids are remapped so that each XCD gets a
// contiguous range of tiles, walked GROUP_M m-tiles at a time so that
// workgroups resident together share their weight and activation tiles.
#include "fp8bs_device.hpp"
#include "fp8bs_internal.hpp"

#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <type_traits>

namespace fp8bs {

constexpr int BK = 128;        // K block = scale block
constexpr int NUM_XCD = 8;     // MI355X: 8 accelerator complex dies
// m-tiles per column sweep: the 32 units an XCD runs at once cover 4 m-tiles x 8
// n-tiles (4 measured 0.6-1.1% faster than 8 over the four 8B-shaped GEMMs; 2
// and 16 slower)
constexpr int GROUP_M = 4;

template <int BM, int BN, int WAVES_M, int WAVES_N>
struct GemmCfg {
    static constexpr int NT = WAVES_M * WAVES_N * 64;
    static constexpr int WM = BM / WAVES_M;
    static constexpr int WN = BN / WAVES_N;
    static constexpr int TM = WM / 16;
    static constexpr int TN = WN / 16;
    static constexpr int ROWS = BM + BN;            // LDS rows per stage: X rows then W rows
    static constexpr int STAGE_BYTES = ROWS * BK;
    static constexpr int CHUNKS = ROWS * (BK / 16); // 16-byte chunks per stage
    static constexpr int LOADS = CHUNKS / NT;       // per thread
    static_assert(CHUNKS % NT == 0, "tile must split evenly over threads");
    static_assert(WM % 16 == 0 && WN % 16 == 0, "wave tile must be made of 16x16 MFMA tiles");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must lie in one 128-wide weight scale block");
};

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// One row tile of the grouped form: `rows` (1 .. BM) rows of expert e from
// row_begin; e < 0 past the last tile.
struct GroupTile {
    int64_t row_begin;
    int32_t e;
    int32_t rows;
};

// Problem description shared by the dense and grouped launches.
struct GemmArgs {
    const uint8_t *xq;
    const float *xs;
    const uint8_t *wq;
    const float *ws;
    const int32_t *offsets; // grouped only
    void *y;
    int64_t M;              // dense: rows; grouped: M_total
    int64_t N, K;
    int64_t E;              // grouped only
    int tiles_m;            // dense: ceil(M/BM); grouped: upper bound ceil(M_total/BM) + E
    int tiles_n;            // N / BN
    int ksplit;             // persistent dense kernel: K ranges per output tile (1 = whole K)
    float *part;            // ksplit > 1: fp32 partial sums [ksplit][M][N]
    const GroupTile *gtab;  // grouped, persistent kernel: the row tiles (tiles_m entries) ...
    const int32_t *gcount;  // ... of which the first *gcount exist
    uint8_t *yq;            // quantizing epilogue: codes [M, N] of the bf16 output ...
    float *ys;              // ... and its 1x128 scales [M, N/128]
};

// Logical tile of workgroup `bid` (XCD-contiguous ranges, GROUP_M swizzle).
__device__ __forceinline__ void tile_of(int bid, int grid, int tiles_m, int tiles_n, int &tm, int &tn)
{
    if (grid % NUM_XCD == 0)
        bid = (bid % NUM_XCD) * (grid / NUM_XCD) + bid / NUM_XCD;
    const int per_group = GROUP_M * tiles_n;
    const int group = bid / per_group;
    const int first_m = group * GROUP_M;
    const int gm = (tiles_m - first_m) < GROUP_M ? (tiles_m - first_m) : GROUP_M;
    const int in = bid % per_group;
    tm = first_m + in % gm;
    tn = in / gm;
}

// Grouped form: which expert owns m-tile `t` of the concatenated per-expert
// tile lists (expert e contributes ceil(count_e / BM) tiles).  Every wave
// computes it from the device offsets, 64 experts per step (one per lane).
// The offsets are clamped into [0, M_total] and made non-decreasing (running
// max), so a malformed table cannot move a row out of bounds.  Returns false
// when t is past the last tile.
template <int BM>
__device__ __forceinline__ bool expert_of_tile(const int32_t *offsets, int64_t E, int64_t M_total, int t, int &e_out,
                                               int64_t &row_begin, int64_t &row_end)
{
    const int lane = threadIdx.x & 63;
    int64_t prev_end = offsets[0];
    prev_end = prev_end < 0 ? 0 : (prev_end > M_total ? M_total : prev_end);
    int base = 0; // tiles of the experts before this step
    for (int64_t e0 = 0; e0 < E; e0 += 64) {
        const int64_t e = e0 + lane;
        int64_t end = (e < E) ? (int64_t)offsets[e + 1] : prev_end;
        end = end < prev_end ? prev_end : (end > M_total ? M_total : end);
        for (int d = 1; d < 64; d <<= 1) { // inclusive max-scan
            const int64_t o = __shfl_up(end, d);
            if (lane >= d && o > end)
                end = o;
        }
        int64_t start = __shfl_up(end, 1);
        if (lane == 0)
            start = prev_end;
        const int cnt = (e < E) ? (int)((end - start + BM - 1) / BM) : 0;
        int inc = cnt; // inclusive prefix sum of the tile counts
        for (int d = 1; d < 64; d <<= 1) {
            const int o = __shfl_up(inc, d);
            if (lane >= d)
                inc += o;
        }
        const int first = base + inc - cnt;
        const unsigned long long hit = __ballot(cnt > 0 && t >= first && t < first + cnt);
        if (hit) {
            const int src = __builtin_ctzll(hit);
            e_out = (int)e0 + src;
            const int64_t s_src = __shfl(start, src), e_src = __shfl(end, src);
            row_begin = s_src + (int64_t)(t - __shfl(first, src)) * BM;
            row_end = (row_begin + BM) < e_src ? (row_begin + BM) : e_src;
            return true;
        }
        base += __shfl(inc, 63);
        prev_end = __shfl(end, 63);
    }
    return false;
}

// The row tiles of the grouped form, written once per launch by one wave so
// that the GEMM workgroups look a tile up with one scalar load.  Expert e's
// rows are cut into BM_A-row tiles from its first row; the last, partial
// tile goes to table B when it has at most BM_B rows (BM_B > 0) -- it is then
// multiplied with BM_B-row tiles instead of padded to BM_A -- and to table A
// otherwise.  Tiles are in expert order; entries past a table's last tile
// get e = -1, and count[0], count[1] receive the two tables' tile counts, so
// that each GEMM spreads exactly the existing tiles over the XCDs.  Offsets
// are clamped and made non-decreasing as in expert_of_tile.  cap_a >=
// ceil(M_total / BM_A) + E and cap_b >= E bound the counts.
template <int BM_A, int BM_B>
__global__ __launch_bounds__(64) void grouped_tile_table_kernel(const int32_t *offsets, int64_t E, int64_t M_total,
                                                                int cap_a, GroupTile *tab_a, int cap_b,
                                                                GroupTile *tab_b, int32_t *count)
{
    const int lane = threadIdx.x;
    int64_t prev_end = offsets[0];
    prev_end = prev_end < 0 ? 0 : (prev_end > M_total ? M_total : prev_end);
    int base_a = 0, base_b = 0;
    for (int64_t e0 = 0; e0 < E; e0 += 64) {
        const int64_t e = e0 + lane;
        int64_t end = (e < E) ? (int64_t)offsets[e + 1] : prev_end;
        end = end < prev_end ? prev_end : (end > M_total ? M_total : end);
        for (int d = 1; d < 64; d <<= 1) { // inclusive max-scan
            const int64_t o = __shfl_up(end, d);
            if (lane >= d && o > end)
                end = o;
        }
        int64_t start = __shfl_up(end, 1);
        if (lane == 0)
            start = prev_end;
        const int64_t rows = (e < E) ? end - start : 0;
        const int64_t rem = rows % BM_A;
        const bool rem_b = BM_B > 0 && rem > 0 && rem <= BM_B;
        const int cnt_a = (int)(rows / BM_A) + ((rem > 0 && !rem_b) ? 1 : 0);
        const int cnt_b = rem_b ? 1 : 0;
        int inc_a = cnt_a, inc_b = cnt_b; // inclusive prefix sums of the tile counts
        for (int d = 1; d < 64; d <<= 1) {
            const int oa = __shfl_up(inc_a, d), ob = __shfl_up(inc_b, d);
            if (lane >= d) {
                inc_a += oa;
                inc_b += ob;
            }
        }
        const int first_a = base_a + inc_a - cnt_a;
        for (int j = 0; j < cnt_a; ++j) {
            const int t = first_a + j;
            const int64_t r0 = start + (int64_t)j * BM_A;
            if (t < cap_a)
                tab_a[t] = GroupTile{r0, (int32_t)e, (int32_t)((end - r0) < BM_A ? (end - r0) : BM_A)};
        }
        if (rem_b) {
            const int t = base_b + inc_b - 1;
            if (t < cap_b)
                tab_b[t] = GroupTile{end - rem, (int32_t)e, (int32_t)rem};
        }
        base_a += __shfl(inc_a, 63);
        base_b += __shfl(inc_b, 63);
        prev_end = __shfl(end, 63);
    }
    for (int t = base_a + lane; t < cap_a; t += 64)
        tab_a[t] = GroupTile{0, -1, 0};
    for (int t = base_b + lane; t < cap_b; t += 64)
        tab_b[t] = GroupTile{0, -1, 0};
    if (lane == 0) {
        count[0] = base_a < cap_a ? base_a : cap_a;
        count[1] = base_b < cap_b ? base_b : cap_b;
    }
}

// WROW: the weight operand carries one scale per row and K block (ws [N, K/128],
// the 1x128 blocks of an activation-like operand: the weight gradient, whose
// both operands are quantized along the tokens), so the scale product differs
// per output column; each lane forms xs * ws for its 4 columns of a tile.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool OUT_F32, bool GROUPED, bool WROW = false>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void gemm_kernel(GemmArgs a)
{
    using C = GemmCfg<BM, BN, WAVES_M, WAVES_N>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * C::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;

    int tm, tn;
    tile_of(blockIdx.x, gridDim.x, a.tiles_m, a.tiles_n, tm, tn);

    int64_t row_begin, row_end; // rows of X / Y this workgroup covers: [row_begin, row_end)
    const uint8_t *wq = a.wq;
    const float *ws = a.ws;
    const int64_t K = a.K, KB = K / BK, N = a.N;
    if (GROUPED) {
        int e;
        if (!expert_of_tile<BM>(a.offsets, a.E, a.M, tm, e, row_begin, row_end))
            return; // past the last tile: uniform over the workgroup
        wq += (int64_t)e * N * K;
        ws += (int64_t)e * (N / 128) * KB;
    } else {
        row_begin = (int64_t)tm * BM;
        row_end = (row_begin + BM) < a.M ? (row_begin + BM) : a.M;
    }
    const int64_t n0 = (int64_t)tn * BN;

    // ---- global -> LDS staging: chunk id -> (LDS row, 16-byte chunk) ----
    const uint8_t *src[C::LOADS];
    int dst[C::LOADS];
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j) {
        const int cid = tid + j * C::NT;
        const int r = cid >> 3, ch = cid & 7;
        if (r < BM) {
            int64_t gr = row_begin + r;
            gr = gr < row_end ? gr : row_end - 1; // rows past the end re-read the last row; never stored
            src[j] = a.xq + gr * K + ch * 16;
        } else {
            src[j] = wq + (n0 + (r - BM)) * K + ch * 16;
        }
        dst[j] = r * BK + ((ch ^ swz(r)) << 4);
    }

    // ---- per-lane fragment addresses (within a stage) ----
    const int fr = lane & 15, fg = lane >> 4; // fragment row, K slice (32 bytes)
    int xoff[C::TM][2], woff[C::TN][2];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int r = wm * C::WM + i * 16 + fr;
        xoff[i][0] = r * BK + (((2 * fg) ^ swz(r)) << 4);
        xoff[i][1] = r * BK + (((2 * fg + 1) ^ swz(r)) << 4);
    }
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
        const int r = BM + wn * C::WN + j * 16 + fr;
        woff[j][0] = r * BK + (((2 * fg) ^ swz(r)) << 4);
        woff[j][1] = r * BK + (((2 * fg + 1) ^ swz(r)) << 4);
    }

    // ---- scale pointers: xs of this lane's rows, ws of this wave's 128 columns ----
    const float *xs_row[C::TM];
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        int64_t gr = row_begin + wm * C::WM + i * 16 + fr;
        gr = gr < row_end ? gr : row_end - 1;
        xs_row[i] = a.xs + gr * KB;
    }
    const float *ws_row = ws + ((n0 + wn * C::WN) / 128) * KB;
    // WROW: the scales of this lane's 4 columns (rows of W) of each n-tile
    const float *ws_col[WROW ? C::TN : 1];
    if constexpr (WROW) {
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            ws_col[j] = ws + (n0 + wn * C::WN + j * 16 + fg * 4) * KB;
    }

    v4f acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    u32x4 stage[C::LOADS];
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j)
        stage[j] = *(const u32x4 *)src[j];
#pragma unroll
    for (int j = 0; j < C::LOADS; ++j)
        *(u32x4 *)(lds + dst[j]) = stage[j];
    __syncthreads();

    for (int64_t kb = 0; kb < KB; ++kb) {
        const int cur = (int)(kb & 1);
        const bool more = kb + 1 < KB;
        if (more) {
#pragma unroll
            for (int j = 0; j < C::LOADS; ++j)
                stage[j] = *(const u32x4 *)(src[j] + (kb + 1) * BK);
        }
        const float sw = WROW ? 1.0f : ws_row[kb];
        float sc[C::TM];
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            sc[i] = xs_row[i][kb] * sw;
        v4f swv[WROW ? C::TN : 1];
        if constexpr (WROW) {
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
                swv[j] = v4f{ws_col[j][kb], ws_col[j][KB + kb], ws_col[j][2 * KB + kb], ws_col[j][3 * KB + kb]};
        }

        const uint8_t *L = lds + cur * C::STAGE_BYTES;
        v8i bx[C::TM], aw[C::TN];
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const u32x4 lo = *(const u32x4 *)(L + xoff[i][0]);
            const u32x4 hi = *(const u32x4 *)(L + xoff[i][1]);
            bx[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const u32x4 lo = *(const u32x4 *)(L + woff[j][0]);
            const u32x4 hi = *(const u32x4 *)(L + woff[j][1]);
            aw[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                // format 0 = FP8 E4M3 for both operands; scale operands 0: the plain (unscaled) MFMA
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[j], bx[i], v4f{0.f, 0.f, 0.f, 0.f},
                                                                               0, 0, 0, 0, 0, 0);
                const v4f scv = v4f{sc[i], sc[i], sc[i], sc[i]};
                if constexpr (WROW)
                    acc[i][j] = __builtin_elementwise_fma(scv * swv[j], p, acc[i][j]);
                else
                    acc[i][j] = __builtin_elementwise_fma(scv, p, acc[i][j]);
            }
        }
        if (more) {
            uint8_t *Ln = lds + (cur ^ 1) * C::STAGE_BYTES;
#pragma unroll
            for (int j = 0; j < C::LOADS; ++j)
                *(u32x4 *)(Ln + dst[j]) = stage[j];
        }
        __syncthreads();
    }

    // ---- epilogue: lane holds Y[m = base + l%16][n = base + 4*(l/16) + 0..3] per MFMA tile ----
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
        const int64_t m = row_begin + wm * C::WM + i * 16 + fr;
        if (m >= row_end)
            continue;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const int64_t n = n0 + wn * C::WN + j * 16 + fg * 4;
            const v4f v = acc[i][j];
            if (OUT_F32) {
                *(v4f *)((float *)a.y + m * N + n) = v;
            } else {
                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                const bf2 p0 = __builtin_convertvector(__builtin_shufflevector(v, v, 0, 1), bf2);
                const bf2 p1 = __builtin_convertvector(__builtin_shufflevector(v, v, 2, 3), bf2);
                *(u32x2 *)((uint16_t *)a.y + m * N + n) =
                    u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
            }
        }
    }
}

// ---- large-tile kernels: direct global->LDS loads -------------------------------
//
// Same product as gemm_kernel, organized for the dense prefill/training
// shapes (M in the thousands) and, split along K, for the few-row ones:
//   - large workgroup tiles, 256 x 256 over 8 waves of 64 x 128 (each wave
//     reads 24 KiB of LDS per 32 MFMAs) or 128 x 256 over 8 waves of 64 x 64,
//     so each K block moves (BM + BN) * 128 bytes for 2 * BM * BN * 128 FLOP.
//     With 8 waves each SIMD holds two, so one wave's fp32 rescale (VALU)
//     runs while the other's MFMAs keep the matrix core busy;
//   - operands and activation scales go from global memory straight into LDS
//     (buffer_load ... lds: each dwordx4 wave instruction fills 1 KiB = 8 LDS
//     rows of 128 bytes, lane i writing bytes 16i .. 16i+15), so no VGPRs or
//     VALU cycles are spent on staging.  The per-lane offset is fixed for the
//     whole loop and the K block advances through the scalar offset;
//   - LDS layout.  A 16-lane group of a ds_read_b128 fragment read touches 16
//     rows at one K chunk; gfx950 serves it without bank conflicts when each
//     8-lane half stays within one 128-byte half of the 256-byte bank space
//     and the 8 lanes of a half hit 8 different 16-byte slots.  So tile row r
//     of each 16-row group lives at LDS row ((r & 7) << 1) | (r >> 3) (rows
//     0-7 on even rows, 8-15 on odd rows) and its 16-byte chunk c at slot
//     c ^ (r & 7).  The LDS position of a DMA lane is fixed by the hardware,
//     so the layout is produced on the global side: the lane that fills LDS
//     row p, slot s fetches the chunk s ^ (r & 7) of the tile row r stored
//     there -- still 8 lanes per 128-byte row, fully coalesced;
//   - STAGES LDS buffers (two for 256 x 256, three for 128 x 256: what fits
//     in 160 KiB): the loads of the next STAGES - 1 K blocks are in flight
//     while a block is multiplied; one barrier per K block both publishes the
//     next block and retires the reads of the buffer the next loads refill.
//     Waits are explicit (s_waitcnt vmcnt with the count of loads issued after
//     the ones needed), with every count a compile-time constant;
//   - the weight scale of a K block is one scalar load; each wave fetches the
//     activation scales of its own 64 rows (one dword per lane) with its
//     operands, into a region of the stage that only it reads;
//   - bf16 output leaves through a per-wave LDS staging area after the
//     stages (16 rows x EPI_CW columns, rows padded by 16 bytes), so each
//     store instruction writes whole 64- or 128-byte row segments instead of
//     16 scattered 32-byte pieces.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES_, bool WROW_ = false>
struct DmaCfg {
    static constexpr int NW = WAVES_M * WAVES_N;
    static constexpr int NT = NW * 64;
    static constexpr int WM = BM / WAVES_M;
    static constexpr int WN = BN / WAVES_N;
    static constexpr int TM = WM / 16;
    static constexpr int TN = WN / 16;
    static constexpr int STAGES = STAGES_;
    static constexpr int XS_OFF = (BM + BN) * BK;            // activation scales after the operand rows
    static constexpr int STAGE_BYTES = XS_OFF + NW * 256;    // 64 fp32 per wave
    static constexpr int XG = BM / 8 / NW; // 1 KiB row groups of X per wave per stage
    static constexpr int WG = BN / 8 / NW; // ... of W
    // LDS-DMA instructions per wave per stage: X and W row groups, activation
    // scales, and (per-row weight scales) the W-row scales
    static constexpr int DPW = XG + WG + 1 + (WROW_ ? 1 : 0);
    // per-row weight scales: a ring of STAGES + 1 slots after the stages, so
    // that the slot a step reads is never the one being refilled while the
    // step still rescales (the refill of step s + STAGES, issued during step s,
    // goes to the slot of step s - 1).  A slot gives each wave 256 bytes: the
    // first BN / 64 waves fetch the BN scales, the others issue the same
    // instruction on an empty range into their own, unread, quarter.
    static constexpr int WSR_SLOTS = WROW_ ? STAGES_ + 1 : 0;
    static constexpr int WSR_STRIDE = NW * 256;
    static constexpr int WSR_OFF = STAGES_ * STAGE_BYTES;
    static constexpr int WSR_BYTES = WSR_SLOTS * WSR_STRIDE;
    static_assert(!WROW_ || BN <= NW * 64, "one W-row scale per lane of the first BN / 64 waves");
    static_assert(STAGES == 2 || STAGES == 3, "two or three LDS stages");
    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "row groups must split evenly over the waves");
    static_assert(BM % 16 == 0, "16-row layout groups must not straddle X and W");
    static_assert(WM == 64, "one activation-scale dword per lane covers the wave's 64 rows");
    static_assert(WN % 16 == 0, "wave tile must be made of 16x16 MFMA tiles");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must lie in one 128-wide weight scale block");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
    // output staging: 64 bf16 columns per row where they fit, else 32
    static constexpr int EPI_CW = STAGES * STAGE_BYTES + WSR_BYTES + NW * 16 * (64 * 2 + 16) <= 160 * 1024 ? 64 : 32;
    static constexpr int EPI_RS = EPI_CW * 2 + 16;
    static constexpr int EPI_BYTES = NW * 16 * EPI_RS;
    static constexpr int EPI_OFF = STAGES * STAGE_BYTES + WSR_BYTES;
    static constexpr int LDS_BYTES = EPI_OFF + EPI_BYTES;
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU (stages and output staging)");
    static_assert(WN % EPI_CW == 0 && EPI_BYTES % 1024 == 0, "output staging chunks");
};

// LDS row of tile row r, and the tile row held by LDS row p (inverse maps).
__device__ __forceinline__ int lds_row(int r) { return (r & ~15) | ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int tile_row(int p) { return (p & ~15) | ((p & 1) << 3) | ((p >> 1) & 7); }

#define LDS_AS __attribute__((address_space(3)))
#define CONST_AS __attribute__((address_space(4)))

// s_waitcnt vmcnt(N) with expcnt / lgkmcnt left alone (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Cache policy of the persistent GEMM's output stores (bf16 Y, the quantizing
// epilogue's codes): nontemporal (the `nt` bit).  Y (67-235 MB per dense GEMM)
// is never read back by the GEMM, while every XCD re-reads the weight panels
// from the 256 MB last-level cache; streamed past the caches, the output no
// longer evicts them.  (The traffic out of the L2s is unchanged, 657 MB per
// launch: what changes is where it is served.)  Measured in the dense layer step
// (M = 8192, a cache-evicting read between launches): step -1.2%, the GEMMs
// 40.3% -> 40.9% of the FP8 peak; MoE gate+up -2.5%; with calls back to back,
// dense gate+up -5.3% and MoE down -12.6%.  Split-K partial sums and the
// quantizing epilogue's scale dwords keep the default policy: the reduction
// reads the partials back at once, and the L2 combines the scattered dwords
// into whole lines.
constexpr int kOutPolicy = 2;

// s_waitcnt lgkmcnt(0) with vmcnt / expcnt left alone.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3:
// 32-bit data format, no swizzle); loads past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes >= 0xffffffffLL ? (int)0xffffffffu : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Geometry of one work unit of the persistent kernels: an output tile and
// the range of K blocks it sums (the whole of K unless the product is split
// along K).
struct TileGeo {
    int64_t row_begin, row_end; // rows of X / Y: [row_begin, row_end)
    int64_t n0;                 // first column of Y (row of W)
    const uint8_t *wq;          // this tile's weight matrix (the expert's, for the grouped form)
    const float *ws;
    int kb0, kb1;               // K blocks [kb0, kb1)
    int ks;                     // index of the K range (0 .. ksplit - 1)
};

// Work unit of virtual id v (< tiles_m * tiles_n * ksplit), or false for a
// grouped tile past the last row tile of its expert list.  Units are spread
// XCD-contiguously; the K range is the slowest index, so the units resident
// on one XCD share the same K slice of both operands.
template <int BM, int BN, bool GROUPED, bool SPLIT>
__device__ __forceinline__ bool tile_geo(const GemmArgs &a, int v, int nunits, TileGeo &g)
{
    {
        // virtual ids v = x (mod 8) run on XCD x (the grid is a multiple of
        // 8); give XCD x the contiguous unit range [x q + min(x, r), ...) of
        // q or q + 1 units, a bijection for any unit count
        const int x = v % NUM_XCD, i = v / NUM_XCD;
        const int q = nunits / NUM_XCD, r = nunits % NUM_XCD;
        v = x * q + (x < r ? x : r) + i;
    }
    const int KB = (int)(a.K / BK);
    if (SPLIT) {
        const int ntl = a.tiles_m * a.tiles_n;
        const int ks = v / ntl;
        v -= ks * ntl;
        g.ks = ks;
        g.kb0 = (int)((int64_t)ks * KB / a.ksplit);
        g.kb1 = (int)((int64_t)(ks + 1) * KB / a.ksplit);
    } else {
        g.ks = 0;
        g.kb0 = 0;
        g.kb1 = KB;
    }
    int tm, tn;
    tile_of(v, 1, a.tiles_m, a.tiles_n, tm, tn); // (grid 1: no second XCD remap)
    g.wq = a.wq;
    g.ws = a.ws;
    if (GROUPED) {
        const CONST_AS GroupTile *d = (const CONST_AS GroupTile *)a.gtab + tm;
        const int e = d->e;
        if (e < 0)
            return false;
        g.row_begin = d->row_begin;
        g.row_end = g.row_begin + d->rows;
        g.wq += (int64_t)e * a.N * a.K;
        g.ws += (int64_t)e * (a.N / 128) * (a.K / BK);
    } else {
        g.row_begin = (int64_t)tm * BM;
        g.row_end = (g.row_begin + BM) < a.M ? (g.row_begin + BM) : a.M;
    }
    g.n0 = (int64_t)tn * BN;
    return true;
}

// Persistent form: gridDim.x workgroups (one per CU) walk the virtual work
// units v = blockIdx.x, blockIdx.x + gridDim.x, ...  All (unit, K block)
// steps of a workgroup form one stream through the LDS stages: the operands
// of step s + STAGES are issued during the last MFMA groups of step s, as
// soon as every wave has finished reading the stage they refill, and the
// fragments of step s + 1 are read into registers during those same groups,
// so the matrix cores never wait on LDS at a step boundary; a unit's output
// stores drain while the next unit computes.  Stores are buffer stores
// whose out-of-range rows the hardware drops.  SPLIT: the work units are
// (tile, K range) pairs and each writes its fp32 partial tile to the
// partial-sum buffer (ksplit slices of M x N), summed by splitk_reduce_kernel.
// POW2: every scale is a power of two (the power-of-2 scale option of the
// article's closing section), so each K block's scale product 2^e is exact
// and goes to the MFMA's E8M0 scale operand: the matrix core accumulates
// 2^e * P into the accumulator itself and the fp32 VALU rescale disappears.
// WROW: per-row weight scales ws [N, K/128] (the weight gradient, whose both
// operands are quantized in 1x128 blocks along the tokens): each K step's BN
// W-row scales travel with its operands into a ring of LDS slots, and the
// rescale forms xs * ws for each lane's 4 columns of a tile; with POW2 each
// lane instead passes the scale of the W row it holds to the MFMA's E8M0
// operand of the weight operand, and both scales reach the matrix core.
// QMODE (1 = EXACT, 2 = POW2 scales): the bf16 output is also quantized in
// 1x128 blocks along its rows, as quant_act_1x128 would quantize it, for a
// next layer that takes FP8 input: codes to a.yq [M, N], scales to a.ys
// [M, N/128]; the bf16 output itself is written only if a.y is not null.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool OUT_F32, bool GROUPED, bool SPLIT, bool POW2,
          bool WROW = false, int QMODE = 0>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void gemm_dma_kernel(GemmArgs args)
{
    static_assert(!(WROW && GROUPED), "per-row weight scales: dense products");
    static_assert(QMODE == 0 || (!OUT_F32 && !SPLIT && !WROW && !GROUPED && BN / WAVES_N == 128),
                  "the quantizing epilogue: bf16 output, whole K, one 128-column block per wave");
    GemmArgs a = args;
    if constexpr (GROUPED)
        a.tiles_m = *(const CONST_AS int32_t *)a.gcount; // the tiles that exist
    // three LDS stages (two steps of loads in flight) where they fit beside
    // the W-row scale ring and the narrower output staging
    using C2 = DmaCfg<BM, BN, WAVES_M, WAVES_N, 2, WROW>;
    constexpr int NST =
        3 * C2::STAGE_BYTES + (WROW ? 4 * C2::WSR_STRIDE : 0) + C2::NW * 16 * (32 * 2 + 16) <= 160 * 1024 ? 3 : 2;
    using C = DmaCfg<BM, BN, WAVES_M, WAVES_N, NST, WROW>;
    // one array: the operand stages, then the output staging area (two
    // separate __shared__ arrays made the main loop run at half speed)
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::LDS_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    const int64_t K = a.K, KB = K / BK, N = a.N;
    const int ntiles = a.tiles_m * a.tiles_n * (SPLIT ? a.ksplit : 1); // work units
    const int sub = lane >> 3, slot = lane & 7;
    const int fr = lane & 15, fg = lane >> 4;
    uint8_t *const epi_lds = lds + C::EPI_OFF + wave * 16 * C::EPI_RS; // this wave's staging rows

    // ---- DMA cursor: the tile and K block whose operands load next ----
    int dv = blockIdx.x;
    TileGeo dt;
    bool dvalid = false;
    while (dv < ntiles && !(dvalid = tile_geo<BM, BN, GROUPED, SPLIT>(a, dv, ntiles, dt)))
        dv += gridDim.x;
    if (!dvalid)
        return; // no tile for this workgroup (uniform)
    TileGeo ct = dt; // tile of the step being computed
    int cv = dv;     // ... and its virtual id
    int64_t dkb = dt.kb0;

    // ---- per-tile DMA state ----
    // Row group t of a wave (LDS rows 8 (wave + NW t) .. + 7) holds tile rows
    // tile_row(8 wave + sub) + 8 NW t: the same per-lane offset for every t,
    // plus 8 NW t rows.  W adds those rows through the scalar offset.  X
    // takes one buffer resource per row group, based at the group's first
    // row and bounded by the tile's last row, so lanes past the end of a
    // ragged tile read zeros through the hardware range check (those rows are
    // never stored); the activation scales are bounded the same way.  Offsets
    // are 32-bit (the launcher only picks this kernel when 256 K < 2^32).
    constexpr int GROW = 8 * C::NW; // rows between a wave's consecutive row groups
    // (the resources are rebuilt per issue from the tile's bases and byte
    // counts, which are computed once per tile: the host pass of this
    // compiler emits no launch stub for a kernel holding an array of buffer
    // resources)
    const uint8_t *xbase, *wbase;
    const float *sbase;
    const float *wrbase = nullptr; // WROW: the tile's W-row scales (rows n0 .. n0 + BN - 1)
    uint32_t xnr[C::XG]; // bytes of X in row group t (0 past the tile's last row)
    uint32_t snr;        // bytes of the tile's activation-scale rows
    const int r0 = tile_row(wave * 8 + sub);
    const uint32_t loff = (uint32_t)(r0 * K) + (uint32_t)((slot ^ (r0 & 7)) << 4);
    const uint32_t soff = (uint32_t)((wm * C::WM + lane) * KB * 4);
    auto dma_setup = [&](const TileGeo &g) {
        xbase = a.xq + g.row_begin * K;
        wbase = g.wq + g.n0 * K;
        sbase = a.xs + g.row_begin * KB;
        if constexpr (WROW)
            wrbase = g.ws + g.n0 * KB;
        const int64_t rows = g.row_end - g.row_begin; // 1 .. BM
#pragma unroll
        for (int t = 0; t < C::XG; ++t) {
            const int64_t left = rows - (int64_t)GROW * t;
            xnr[t] = left > 0 ? (uint32_t)(left * K) : 0u;
        }
        snr = (uint32_t)(rows * KB * 4);
    };
    // Load q (0 .. DPW - 1) of K block kb into `stage`: X row groups, then W
    // row groups, then the activation scales.  With live == false every
    // range is empty, so the same instructions move nothing (the hardware
    // range check drops them): the caller issues them unconditionally,
    // keeping the MFMA stream they sit in free of branches.
    auto issue_q = [&](int q, int64_t kb, int stage, int wslot, bool live) __attribute__((always_inline)) {
        uint8_t *L = lds + stage * C::STAGE_BYTES;
        const int ko = (int)(kb * BK);
        if (WROW && q == C::XG + C::WG + 1) {
            // W-row scales of K block kb: lane l of wave w < BN / 64 fetches row
            // 64 w + l into its quarter of slot `wslot`; the other waves issue
            // on an empty range into their own quarters, which nothing reads
            const bool mine = wave < BN / 64;
            const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float *>(wrbase), (short)0, (live && mine) ? (int)(BN * KB * 4) : 0, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                wr, (LDS_AS void *)(lds + C::WSR_OFF + wslot * C::WSR_STRIDE + wave * 256), 4,
                (int)((uint32_t)((mine ? wave * 64 + lane : 0) * KB * 4)), (int)(kb * 4), 0, 0);
            return;
        }
        if (q < C::XG) {
            const int t = q;
            const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(xbase + (int64_t)GROW * t * K), (short)0, (int)(live ? xnr[t] : 0u), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (LDS_AS void *)(L + (wave + C::NW * t) * 1024), 16,
                                                     (int)loff, ko, 0, 0);
        } else if (q < C::XG + C::WG) {
            const int t = q - C::XG;
            const __amdgpu_buffer_rsrc_t wl = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(wbase), (short)0, live ? (int)(uint32_t)((int64_t)BN * K) : 0, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wl, (LDS_AS void *)(L + BM * BK + (wave + C::NW * t) * 1024),
                                                     16, (int)loff, ko + (int)(GROW * t * K), 0, 0);
        } else {
            const __amdgpu_buffer_rsrc_t sl = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float *>(sbase), (short)0, (int)(live ? snr : 0u), 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(sl, (LDS_AS void *)(L + C::XS_OFF + wave * 256), 4, (int)soff,
                                                     (int)(kb * 4), 0, 0);
        }
    };
    auto issue = [&](int64_t kb, int stage, bool live = true) {
        // (the prologue's steps 0 .. STAGES - 1 use W-row slots 0 .. STAGES - 1)
#pragma unroll
        for (int q = 0; q < C::DPW; ++q)
            issue_q(q, kb, stage, stage, live);
    };
    // advance the DMA cursor by one K block; false at the end of the stream
    auto dma_next = [&]() {
        if (++dkb < dt.kb1)
            return true;
        do {
            dv += gridDim.x;
        } while (dv < ntiles && !tile_geo<BM, BN, GROUPED, SPLIT>(a, dv, ntiles, dt));
        if (dv >= ntiles)
            return false;
        dma_setup(dt);
        dkb = dt.kb0;
        return true;
    };

    // ---- fragment offsets within a stage ----
    // Lane l reads tile row (l % 16) of a 16-row MFMA tile, K chunks 2 (l/16)
    // and 2 (l/16) + 1; consecutive MFMA tiles are 2048 bytes apart, so one
    // base per operand half plus immediates covers every fragment.
    int xo[2], wo[2];
    {
        const int px = (wm * C::WM + lds_row(fr)) * BK, pw = (BM + wn * C::WN + lds_row(fr)) * BK;
        xo[0] = px + (((2 * fg) ^ (fr & 7)) << 4);
        xo[1] = px + (((2 * fg + 1) ^ (fr & 7)) << 4);
        wo[0] = pw + (((2 * fg) ^ (fr & 7)) << 4);
        wo[1] = pw + (((2 * fg + 1) ^ (fr & 7)) << 4);
    }
    const int so = C::XS_OFF + wave * 256 + fr * 4;

    v4f acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    auto frag = [](const uint8_t *p0, const uint8_t *p1) {
        const u32x4 lo = *(const u32x4 *)p0;
        const u32x4 hi = *(const u32x4 *)p1;
        return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    };

    // Fragments and scale products of the step being computed.  Except for
    // the first step they are read from the step's LDS stage while the
    // previous step's last WD MFMA groups run.  W fragments rotate through a
    // ring of WD + 1 (the group being multiplied and the next WD).  WD = 3
    // where a step has 8 groups: each fragment read then has three groups
    // of MFMAs to land instead of two, which made the 256x256 products
    // 1.7-3.3% faster with bit-identical results.  Products with 4 groups a
    // step (the 64- and 128-row tiles) showed no gain, and the fp32-output
    // EXACT form with per-row weight scales would spill more; they keep
    // WD = 2.
    constexpr bool DEEP = C::TN >= 8 && !(WROW && OUT_F32 && !POW2);
    constexpr int WD = DEEP ? 3 : 2, WR = WD + 1;
    v8i bx[C::TM];
    v8i awq[WR];
    float sc[C::TM];   // the step's scale product per row tile (POW2: the activation scale alone)
    float sw_cur = 1.f; // the step's weight scale (POW2)
    auto ws_of = [&](const TileGeo &g) {
        return (const CONST_AS float *)(g.ws + ((g.n0 + wn * C::WN) / 128) * KB);
    };
    auto sync = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // WROW: this lane's 4 W-row scales of n-tile j, in slot j % 2 (read at the
    // start of group j; group j's last rescale runs in group j + 1)
    v4f wsv[2];
    auto rescale = [&](int t, const v4f &p) {
        const int i = t % C::TM, j = t / C::TM;
        if constexpr (WROW)
            acc[i][j] = __builtin_elementwise_fma(v4f{sc[i], sc[i], sc[i], sc[i]} * wsv[j & 1], p, acc[i][j]);
        else
            acc[i][j] = __builtin_elementwise_fma(v4f{sc[i], sc[i], sc[i], sc[i]}, p, acc[i][j]);
    };
    static_assert(C::TN >= 4, "the W-fragment ring needs at least four groups per step");

    // One K block from registers.  Group j (TM MFMAs on one W fragment)
    // reads the W fragment of group j + WD, so each LDS read has WD groups of
    // MFMAs to land.  The rescale of MFMA tile t is issued after the MFMA of
    // tile t + 1, so the matrix core has the next product queued while the
    // VALU applies the previous one.  Before group TN - WD every wave waits
    // for the next step's operands and for its own LDS reads (the last read
    // of this stage was issued in group TN - WD - 1), and passes the barrier:
    // the next stage is then complete for all waves and no wave reads this
    // stage any more, so the loads of a later step may refill it.  Those
    // loads are spread over the MFMAs of the last WD groups (issued in one
    // block right after the barrier, where every wave of the CU is at the
    // same point, they would leave the matrix cores idle while their
    // addresses are formed).  The last WD groups also read the next step's
    // first WD W fragments and its scales, and each MFMA of the last group
    // frees its X fragment registers for the next step's.  (For the last
    // step of a workgroup those reads fetch data that is never used; the
    // barrier is uniform.)
    auto compute = [&](int stage, int nstage, int wcur, bool full_wait, const CONST_AS float *swp, auto &&load_q)
                       __attribute__((always_inline)) {
        const uint8_t *L = lds + stage * C::STAGE_BYTES;
        const uint8_t *Ln = lds + nstage * C::STAGE_BYTES;
        const uint8_t *Lw = lds + C::WSR_OFF + wcur * C::WSR_STRIDE + (wn * C::WN + 4 * fg) * 4;
        // (POW2 with per-row weight scales: the scale of W row fr of each 16-row tile, this lane's
        // row of the MFMA's weight operand)
        const uint8_t *Lwe = lds + C::WSR_OFF + wcur * C::WSR_STRIDE + (wn * C::WN + fr) * 4;
        v4f part[2];
        float xs_next[C::TM];
        float sw_next = 0.f;
        // POW2: each factor of the scale product goes to its own operand's
        // E8M0 scale, as its biased exponent (exact for every power of two
        // from 2^-127 up; the product itself may lie below fp32's normal
        // range): the step's weight scale on the weight operand, uniform over
        // the wave, and the activation row's scale on the activation operand --
        // lane l holds the fragment of row l % 16, whose scale it passes.
        int e8[C::TM];
        int e8w = 127;
        if constexpr (POW2) {
#pragma unroll
            for (int i = 0; i < C::TM; ++i)
                e8[i] = (int)(__builtin_bit_cast(uint32_t, sc[i]) >> 23);
            e8w = (int)(__builtin_bit_cast(uint32_t, sw_cur) >> 23);
        }
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const bool last = j + 1 == C::TN;
            // (issued before the group's fragment reads: LDS reads complete in
            // order, so waiting for it leaves those in flight)
            int e8wj = e8w;
            if constexpr (WROW && POW2)
                e8wj = (int)(__builtin_bit_cast(uint32_t, *(const float *)(Lwe + j * 64)) >> 23);
            else if constexpr (WROW)
                wsv[j & 1] = *(const v4f *)(Lw + j * 64);
            if (j + WD < C::TN) {
                awq[(j + WD) % WR] = frag(L + wo[0] + (j + WD) * 2048, L + wo[1] + (j + WD) * 2048);
            } else if (j + WD == C::TN) {
                // the next step's loads have landed; those of the steps after
                // it (issued later) may still fly.  The count also covers
                // stores, which may complete out of order with the loads: in
                // the first step after a tile's output stores, wait for all.
                if (C::STAGES == 2 || full_wait)
                    wait_vmcnt<0>();
                else
                    wait_vmcnt<(C::STAGES - 2) * C::DPW>();
                wait_lgkmcnt0();
                sync();
                // the next step's weight scale (a valid address even past the
                // end of the stream, where the value goes unused): no wait for
                // an LDS read falls between here and the end of the step, where
                // the reads issued below are waited for anyway, so the scalar
                // load's out-of-order return costs nothing
                if constexpr (!WROW)
                    sw_next = *swp;
                else
                    sw_next = 1.0f; // (the weight scale is applied per column)
                awq[(j + WD) % WR] = frag(Ln + wo[0], Ln + wo[1]);
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
                    xs_next[i] = *(const float *)(Ln + so + i * 64);
            } else {
                awq[(j + WD) % WR] = frag(Ln + wo[0] + (j + WD - C::TN) * 2048, Ln + wo[1] + (j + WD - C::TN) * 2048);
            }
            // the reads above stay ahead of this group's MFMAs (the machine
            // scheduler would otherwise sink them to where the registers they
            // fill are next used, shrinking the prefetch distance to zero)
            __builtin_amdgcn_sched_barrier(0);
            const v8i aw = awq[j % WR];
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                const int t = j * C::TM + i;
                if constexpr (POW2)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, bx[i], acc[i][j], 0, 0, 0, e8wj, 0,
                                                                                 e8[i]);
                else
                    part[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        aw, bx[i], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                // issue order: each MFMA, then the rescale of the previous
                // one (whose product has had a full MFMA to land), and in the
                // last group the next step's X fragment it freed; after the
                // barrier, the next loads one or two per MFMA.  Only the last
                // WD groups, which carry the loads, are fenced per MFMA;
                // elsewhere the scheduler may interleave MFMAs and rescales
                // (about 1% faster than fencing every MFMA)
                if (j + WD >= C::TN)
                    __builtin_amdgcn_sched_barrier(0);
                if (!POW2 && t > 0)
                    rescale(t - 1, part[(t - 1) & 1]);
                if (last)
                    bx[i] = frag(Ln + xo[0] + i * 2048, Ln + xo[1] + i * 2048);
                if (j + WD >= C::TN) {
                    const int slot_i = (j + WD - C::TN) * C::TM + i;
#pragma unroll
                    for (int q = 0; q < C::DPW; ++q)
                        if (q * WD * C::TM / C::DPW == slot_i)
                            load_q(q);
                }
                if (j + WD >= C::TN)
                    __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (!POW2)
            rescale(C::TM * C::TN - 1, part[(C::TM * C::TN - 1) & 1]);
        // (POW2 keeps the two factors apart for the E8M0 operands)
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            sc[i] = POW2 ? xs_next[i] : xs_next[i] * sw_next;
        sw_cur = sw_next;
        // the next step's groups 0 .. WD - 1 were read into slots (TN + t) % WR;
        // move them to slots 0 .. WD - 1 (nothing to move when TN % WR == 0)
        if constexpr (C::TN % WR != 0) {
            v8i nx[WD];
#pragma unroll
            for (int t = 0; t < WD; ++t)
                nx[t] = awq[(C::TN + t) % WR];
#pragma unroll
            for (int t = 0; t < WD; ++t)
                awq[t] = nx[t];
        }
    };

    // Output of a finished work unit: buffer stores over the tile's own rows,
    // so rows past row_end are dropped by the range check, not by a branch.
    // A unit that sums one K range of a split product writes its fp32
    // partial tile to slice ks of the partial-sum buffer instead.
    auto store = [&](auto f32_tag, const uint8_t *base, const TileGeo &g) {
        constexpr bool F32 = decltype(f32_tag)::value;
        constexpr int ES = F32 ? 4 : 2;
        const int64_t rows = g.row_end - g.row_begin;
        const bool want_y = QMODE == 0 || base != nullptr;
        const __amdgpu_buffer_rsrc_t yr =
            make_rsrc(want_y ? base + (g.row_begin * N + g.n0) * ES : (const uint8_t *)a.yq, want_y ? rows * N * ES : 0);
        if constexpr (!F32) {
            // per 16-row tile and EPI_CW-column chunk: each lane writes its 4
            // columns of each MFMA tile into the wave's staging rows, then reads
            // back 16 contiguous bytes of one row, so LPR lanes cover a whole
            // row segment of the store (LDS reads and writes of one wave
            // complete in order, so no barrier is needed)
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
            constexpr int LPR = C::EPI_CW * 2 / 16; // lanes per staged row
            constexpr int RPI = 64 / LPR;           // rows per read-back
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                // the tile's bf16 values (round to nearest even), as pairs of
                // dwords: lane l holds columns 4 (l / 16) .. + 3 of every
                // 16-column tile j of row l % 16 (recomputed per pass: a
                // conversion costs less than the registers of a copy)
                auto bw_of = [&](int j) {
                    const v4f v = acc[i][j];
                    const bf2 p0 = __builtin_convertvector(__builtin_shufflevector(v, v, 0, 1), bf2);
                    const bf2 p1 = __builtin_convertvector(__builtin_shufflevector(v, v, 2, 3), bf2);
                    return u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
                };
                if constexpr (QMODE != 0) {
                    // Row l % 16's 128 columns of this wave are one 1x128 block of
                    // the next layer's input, held by the four lanes l % 16 + 16 q:
                    // amax over the lane's 32 values, then across those lanes; the
                    // scale and codes follow the activation quantizer's encoder, so
                    // they equal quant_act_1x128 of the bf16 output bit for bit.
                    constexpr int QM = QMODE == 2 ? SCALE_POW2 : SCALE_EXACT;
                    uint32_t mx = 0;
#pragma unroll
                    for (int j = 0; j < C::TN; ++j) {
                        const u32x2 w = bw_of(j);
                        const uint32_t a0 = w.x & 0x7fff7fffu, a1 = w.y & 0x7fff7fffu;
                        const uint32_t m0 = (a0 & 0xffffu) > (a0 >> 16) ? (a0 & 0xffffu) : (a0 >> 16);
                        const uint32_t m1 = (a1 & 0xffffu) > (a1 >> 16) ? (a1 & 0xffffu) : (a1 >> 16);
                        const uint32_t m01 = m0 > m1 ? m0 : m1;
                        mx = mx > m01 ? mx : m01;
                    }
                    uint32_t o = (uint32_t)__shfl_xor((int)mx, 16);
                    mx = mx > o ? mx : o;
                    o = (uint32_t)__shfl_xor((int)mx, 32);
                    mx = mx > o ? mx : o;
                    BlockQuant<QM> bq;
                    bq.init(amax_value(mx));
                    // codes staged by rows (row fr: bytes 16 j + 4 fg), then read back
                    // 16 bytes per lane, 8 lanes per 128-byte row
                    // one wave-uniform test for the rare blocks outside the fast
                    // quotient's window (then every lane takes IEEE division,
                    // which is exact for all), instead of a divergent branch per
                    // call: it keeps the epilogue's code, and its share of the
                    // instruction cache, small
                    if (__builtin_amdgcn_ballot_w64(!bq.fast) == 0) {
#pragma unroll
                        for (int j = 0; j < C::TN; ++j) {
                            const u32x2 w = bw_of(j);
                            *(uint32_t *)(epi_lds + fr * C::EPI_RS + j * 16 + fg * 4) =
                                quant4_fast<QM>(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y), bq);
                        }
                    } else {
#pragma unroll
                        for (int j = 0; j < C::TN; ++j) {
                            const u32x2 w = bw_of(j);
                            *(uint32_t *)(epi_lds + fr * C::EPI_RS + j * 16 + fg * 4) =
                                quant4_ieee(bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y), bq.s);
                        }
                    }
                    const __amdgpu_buffer_rsrc_t qr = make_rsrc(a.yq + g.row_begin * N + g.n0, rows * N);
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int r = h * 8 + lane / 8, cc = lane % 8;
                        const u32x4 d = *(const u32x4 *)(epi_lds + r * C::EPI_RS + cc * 16);
                        const int m = wm * C::WM + i * 16 + r;
                        __builtin_amdgcn_raw_buffer_store_b128(d, qr, (int)((int64_t)m * N + wn * C::WN + cc * 16), 0,
                                                               kOutPolicy);
                    }
                    const int64_t NB = N / 128;
                    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.ys + g.row_begin * NB, rows * NB * 4);
                    if (fg == 0)
                        __builtin_amdgcn_raw_buffer_store_b32(
                            __builtin_bit_cast(uint32_t, bq.s), sr,
                            (int)(((int64_t)(wm * C::WM + i * 16 + fr) * NB + g.n0 / 128 + wn) * 4), 0, 0);
                }
                if (want_y) {
#pragma unroll
                for (int c = 0; c < C::WN / C::EPI_CW; ++c) {
#pragma unroll
                    for (int jj = 0; jj < C::EPI_CW / 16; ++jj)
                        *(u32x2 *)(epi_lds + fr * C::EPI_RS + jj * 32 + fg * 8) = bw_of(c * (C::EPI_CW / 16) + jj);
#pragma unroll
                    for (int h = 0; h < 16 / RPI; ++h) {
                        const int r = h * RPI + lane / LPR, cc = lane % LPR;
                        const u32x4 d = *(const u32x4 *)(epi_lds + r * C::EPI_RS + cc * 16);
                        const int m = wm * C::WM + i * 16 + r;
                        const int n = wn * C::WN + c * C::EPI_CW + cc * 8;
                        __builtin_amdgcn_raw_buffer_store_b128(d, yr, (int)(((int64_t)m * N + n) * 2), 0, kOutPolicy);
                    }
                }
                }
#pragma unroll
                for (int j = 0; j < C::TN; ++j)
                    acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int m = wm * C::WM + i * 16 + fr;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int n = wn * C::WN + j * 16 + fg * 4;
                const int off = (int)(((int64_t)m * N + n) * ES);
                // fp32 (a split product's partial tile, or fp32 output): each
                // lane's 16 bytes, 4 lanes per 64-byte row segment
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), yr, off, 0, 0);
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto epilogue = [&](const TileGeo &g) {
        if constexpr (SPLIT)
            store(std::true_type{}, (const uint8_t *)(a.part + (int64_t)g.ks * a.M * N), g);
        else
            store(std::integral_constant<bool, OUT_F32>{}, (const uint8_t *)a.y, g);
    };

    // Pipeline.  While step s is computed from stage s % STAGES, the loads of
    // steps s + 1 .. s + STAGES - 1 are in flight (or landed) in the other
    // stages; those of step s + STAGES are issued after the barrier near the
    // end of step s, the earliest point at which every wave has finished
    // reading the stage they refill.  Every pipeline slot issues its
    // loads -- on empty ranges past the end of the stream -- so the wait
    // counts stay exact.  Per step in flight only a flag and the address of
    // its weight scale are carried; the tile of the step being computed
    // advances with its own cursor.
    // prologue: steps 0 .. STAGES - 2 issued, step 0's fragments and scales read
    dma_setup(dt);
    issue(dkb, 0);
    bool dmore = dma_next();
    const bool has1_0 = dmore;
    const CONST_AS float *wsp1_0 = has1_0 ? ws_of(dt) + dkb : ws_of(ct) + ct.kb0;
    bool has2 = false; // (three stages) step s + 2 exists
    const CONST_AS float *wsp2 = wsp1_0;
    if constexpr (C::STAGES == 3) {
        issue(dkb, 1, has1_0);
        if (has1_0)
            dmore = dma_next();
        has2 = has1_0 && dmore;
        wsp2 = has2 ? ws_of(dt) + dkb : wsp1_0;
    }
    wait_vmcnt<(C::STAGES - 2) * C::DPW>();
    sync();
    {
        const float sw = WROW ? 1.0f : ws_of(ct)[ct.kb0];
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            sc[i] = POW2 ? *(const float *)(lds + so + i * 64) : *(const float *)(lds + so + i * 64) * sw;
        sw_cur = sw;
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            bx[i] = frag(lds + xo[0] + i * 2048, lds + xo[1] + i * 2048);
#pragma unroll
        for (int t = 0; t < WD; ++t)
            awq[t] = frag(lds + wo[0] + t * 2048, lds + wo[1] + t * 2048);
    }
    bool has1 = has1_0;
    const CONST_AS float *wsp1 = wsp1_0;
    {
        // the last slot: step STAGES - 1 into stage STAGES - 1
        const bool hl = C::STAGES == 3 ? has2 : has1;
        issue(dkb, C::STAGES - 1, hl);
        if (hl)
            dmore = dma_next();
    }

    int stage = 0;
    int wcur = 0; // W-row scale slot of the step being computed (WROW)
    int64_t ckb = ct.kb0;
    bool advance = false; // the cursor's step was issued during the previous step
    bool stored = false;  // the previous step ended with a tile's output stores
    while (true) {
        if (advance)
            dmore = dma_next();
        const bool hasS = dmore; // step s + STAGES exists
        const int64_t kbS = dkb;
        const CONST_AS float *wspS = hasS ? ws_of(dt) + dkb : (C::STAGES == 3 ? wsp2 : wsp1);
        const int nstage = stage + 1 == C::STAGES ? 0 : stage + 1;
        // only the loads go in the middle of the MFMA stream; the cursor
        // advances (and sets up the next tile's loads) at the top of the
        // next step
        // step s + STAGES refills the W-row slot of step s - 1
        const int wslotS = wcur == 0 ? C::STAGES : wcur - 1;
        compute(stage, nstage, wcur, stored, wsp1, [&](int q) { issue_q(q, kbS, stage, wslotS, hasS); });
        advance = hasS;
        stage = nstage;
        wcur = wcur == C::STAGES ? 0 : wcur + 1;
        stored = false;
        if (++ckb == ct.kb1) {
            epilogue(ct);
            stored = true;
            if (has1) {
                do {
                    cv += gridDim.x;
                } while (!tile_geo<BM, BN, GROUPED, SPLIT>(a, cv, ntiles, ct));
                ckb = ct.kb0;
            }
        }
        if (!has1)
            break;
        if constexpr (C::STAGES == 3) {
            has1 = has2;
            wsp1 = wsp2;
            has2 = hasS;
            wsp2 = wspS;
        } else {
            has1 = hasS;
            wsp1 = wspS;
        }
    }
}

// ---- weight-streaming kernel for few activation rows (rollout decode) ------------
//
// With M <= 256 the product is bound by reading W from HBM.  A
// workgroup owns TN * 16 rows of W and TM * 16 rows of X (blockIdx.y walks
// the row chunks of X); its 8 waves split the K blocks (wave w takes blocks
// w, w + 8, ...), so every W byte is loaded by exactly one wave, straight
// from global memory into MFMA operand registers with D blocks in flight:
// no LDS and no barrier in the main loop.  X rows past M read as zeros
// through the buffer range check, and their scales as zeros.  At the end the
// 8 per-wave partial tiles are summed through LDS in wave order (a fixed
// order, so results are deterministic) and written out.
constexpr int kSkinnyMaxIt = 16; // K blocks per wave of the weight-streaming kernel (K <= 16384)

//
// QX = 0: X arrives quantized (a.xq codes, a.xs scales).  QX = 1 / 2: a.xq
// holds bf16 activations, and each wave quantizes the fragments it loads with
// the 1x128 activation quantizer's own encoder (EXACT / POW2 scales): a
// lane's 32 consecutive K values of one row are a quarter of a 128-value
// block, whose other quarters sit 16 and 32 lanes away, so two lane
// exchanges give the block's amax.  The codes and scales are bit for bit
// those quant_act_1x128 writes, so Y is that of quant_act_1x128 followed by
// this kernel.
template <int TM, int TN, int D, bool OUT_F32, int QX>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(GemmArgs a)
{
    constexpr int NW = 8;
    constexpr int XB = QX ? 2 : 1; // bytes per X element as loaded
    // loads per K block: W lo/hi, X (lo/hi and a scale, or four bf16 chunks), W scale
    constexpr int LPB = 2 * TN + (QX ? 4 * TM : 3 * TM) + 1;
    static_assert((D - 1) * LPB < 64, "outstanding loads must fit the vmcnt field");
    // (rows padded by 16 bytes: the 16 rows a 16-lane group writes then fall
    // in different banks)
    __shared__ __attribute__((aligned(16))) float red[NW][TM * 16][TN * 16 + 4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int fr = lane & 15, fg = lane >> 4;
    const int64_t K = a.K, KB = K / BK, N = a.N, M = a.M;
    const int64_t n0 = (int64_t)blockIdx.x * (TN * 16);
    const int64_t m0 = (int64_t)blockIdx.y * (TM * 16);
    const int64_t mrows = (M - m0) < TM * 16 ? (M - m0) : TM * 16;

    // W rows n0 .. n0 + 16 TN - 1 (all inside W: N % (16 TN) == 0); X rows
    // m0 .. m0 + mrows - 1.  Lane offsets: row fr of a 16-row tile, bytes
    // 32 fg .. 32 fg + 31 of the K block (the same K order for both operands).
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(a.wq + n0 * K, (int64_t)TN * 16 * K);
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.xq + m0 * K * XB, mrows * K * XB);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.xs + m0 * KB, mrows * KB * 4);
    const __amdgpu_buffer_rsrc_t none = make_rsrc(a.xq, 0);
    // the weight scales of this tile's 128-row block, loaded with the operands
    // (one uniform dword per K block) so that no scalar-load wait sits among
    // the MFMAs
    const __amdgpu_buffer_rsrc_t wsr = make_rsrc(a.ws + (n0 / 128) * KB, KB * 4);
    const int loff = (int)(fr * K + fg * 32);
    const int soff = (int)(fr * KB * 4);

    const int nk = wave < KB ? (int)((KB - wave + NW - 1) / NW) : 0; // this wave's K blocks

    v8i wf[D][TN], xf[D][TM];
    float xv[D][TM], wv[D];
    u32x4 xb[QX ? D : 1][TM][4]; // bf16 X: bytes 64 fg .. 64 fg + 63 of the row's K block
    // Loads of this wave's it-th K block into ring slot `slot`.  Blocks past
    // the end issue the same instructions on an empty range (no traffic), so
    // every step issues LPB loads and the waits below are fixed counts.
    auto load = [&](int slot, int it) {
        const bool live = it < nk;
        const int kb = live ? (int)(wave + (int64_t)it * NW) : 0;
        const __amdgpu_buffer_rsrc_t w_ = live ? wr : none, x_ = live ? xr : none, s_ = live ? sr : none,
                                     t_ = live ? wsr : none;
        wv[slot] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(t_, 0, kb * 4, 0));
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int so = kb * BK + (int)(j * 16 * K);
            const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(w_, loff, so, 0);
            const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(w_, loff + 16, so, 0);
            wf[slot][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        // (the X row of a lane is in the per-lane offset, so a row past M
        // is out of range however the hardware counts the scalar offset)
        if constexpr (QX) {
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int vo = 2 * loff + (int)(i * 16 * K * 2);
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    xb[slot][i][c] = __builtin_amdgcn_raw_buffer_load_b128(x_, vo + 16 * c, kb * BK * 2, 0);
            }
            return;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int vo = loff + (int)(i * 16 * K);
            const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(x_, vo, kb * BK, 0);
            const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(x_, vo + 16, kb * BK, 0);
            xf[slot][i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            xv[slot][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                        s_, soff + (int)(i * 16 * KB * 4), kb * 4, 0));
        }
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // The K loop is unrolled completely (a wave has at most kSkinnyMaxIt
    // blocks; the launcher guarantees it), so the compiler sees which loads
    // are in flight at every wait: a rolled loop made it drain all of them
    // at the loop head.
#pragma unroll
    for (int d = 0; d < D; ++d)
        load(d, d);
#pragma unroll
    for (int it = 0; it < kSkinnyMaxIt; ++it) {
        const int d = it % D;
        wait_vmcnt<(D - 1) * LPB>(); // block `it` landed; D - 1 younger blocks may fly
        if constexpr (QX) {
            constexpr int MODE = QX - 1;
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                uint32_t mag = chunk_max_mag(xb[d][i][0]);
#pragma unroll
                for (int c = 1; c < 4; ++c) {
                    const uint32_t m = chunk_max_mag(xb[d][i][c]);
                    mag = mag > m ? mag : m;
                }
                uint32_t o = (uint32_t)__shfl_xor((int)mag, 16);
                mag = mag > o ? mag : o;
                o = (uint32_t)__shfl_xor((int)mag, 32);
                mag = mag > o ? mag : o;
                BlockQuant<MODE> bq;
                bq.init(amax_value(mag));
                const u32x2 c0 = quant_chunk<MODE>(xb[d][i][0], bq), c1 = quant_chunk<MODE>(xb[d][i][1], bq);
                const u32x2 c2 = quant_chunk<MODE>(xb[d][i][2], bq), c3 = quant_chunk<MODE>(xb[d][i][3], bq);
                xf[d][i] = v8i{(int)c0.x, (int)c0.y, (int)c1.x, (int)c1.y, (int)c2.x, (int)c2.y, (int)c3.x, (int)c3.y};
                xv[d][i] = bq.s;
            }
        }
        const float sw = wv[d];
        float sc[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            sc[i] = xv[d][i] * sw;
        v4f part[2];
#pragma unroll
        for (int t = 0; t < TM * TN; ++t) {
            const int i = t % TM, j = t / TM;
            part[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[d][j], xf[d][i], v4f{0.f, 0.f, 0.f, 0.f},
                                                                           0, 0, 0, 0, 0, 0);
            if (t > 0) {
                const int pi = (t - 1) % TM, pj = (t - 1) / TM;
                acc[pi][pj] = __builtin_elementwise_fma(v4f{sc[pi], sc[pi], sc[pi], sc[pi]}, part[(t - 1) & 1],
                                                        acc[pi][pj]);
            }
        }
        constexpr int T = TM * TN;
        acc[TM - 1][TN - 1] = __builtin_elementwise_fma(v4f{sc[TM - 1], sc[TM - 1], sc[TM - 1], sc[TM - 1]},
                                                        part[(T - 1) & 1], acc[TM - 1][TN - 1]);
        if (it + 1 >= nk)
            break; // (uniform over the wave; later blocks are past this wave's share)
        load(d, it + D);
    }
    wait_vmcnt<0>();

    // ---- sum the 8 waves' partial tiles (wave order) and store ----
    // lane holds Y[m = 16 i + fr][n = 16 j + 4 fg .. + 3] of its partial tile
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
            *(v4f *)&red[wave][i * 16 + fr][j * 16 + fg * 4] = acc[i][j];
    __syncthreads();
    constexpr int GROUPS = TM * 16 * TN * 4; // 4-column groups of the tile
    for (int g = threadIdx.x; g < GROUPS; g += NW * 64) {
        const int m = g / (TN * 4), n = (g % (TN * 4)) * 4;
        v4f v = *(const v4f *)&red[0][m][n];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            v += *(const v4f *)&red[w][m][n];
        if (m < mrows) {
            const int64_t row = m0 + m, col = n0 + n;
            if (OUT_F32) {
                *(v4f *)((float *)a.y + row * N + col) = v;
            } else {
                typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                const bf2 p0 = __builtin_convertvector(__builtin_shufflevector(v, v, 0, 1), bf2);
                const bf2 p1 = __builtin_convertvector(__builtin_shufflevector(v, v, 2, 3), bf2);
                *(u32x2 *)((uint16_t *)a.y + row * N + col) =
                    u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
            }
        }
    }
}

// ---- split-K reduction ----------------------------------------------------------
//
// Y = sum over the K ranges of the fp32 partial tiles, added in K-range order
// (a fixed order, so results are deterministic), four columns per thread.
// The loads of up to 8 ranges are issued before their sum.
template <bool OUT_F32>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float *__restrict__ part, void *__restrict__ y,
                                                            int64_t MN, int ksplit)
{
    const int64_t n4 = MN / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        v4f v = *(const v4f *)(part + i * 4);
        for (int s = 1; s < ksplit; s += 8) {
            v4f t[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s + u < ksplit)
                    t[u] = *(const v4f *)(part + (s + u) * MN + i * 4);
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (s + u < ksplit)
                    v += t[u];
        }
        if (OUT_F32) {
            *(v4f *)((float *)y + i * 4) = v;
        } else {
            typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
            const bf2 p0 = __builtin_convertvector(__builtin_shufflevector(v, v, 0, 1), bf2);
            const bf2 p1 = __builtin_convertvector(__builtin_shufflevector(v, v, 2, 3), bf2);
            *(u32x2 *)((uint16_t *)y + i * 4) = u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
        }
    }
}

// ---- variant table -----------------------------------------------------------------
//
// A shape picks its kernel from (M, N, K) alone -- never from out_dtype -- so
// the fp32 and bf16 outputs of one shape come from the same arithmetic.
// For measurements, FP8BS_GEMM_VARIANT=simple|dma|dma8|skinny forces a kernel
// where its shape constraints allow (dma: 128 x 256 tiles, dma8: 256 x 256)
// and FP8BS_GEMM_KSPLIT=n the number of K ranges of the persistent dense
// kernel; both are read once per process.

enum Variant { V_AUTO = 0, V_SIMPLE = 1, V_DMA = 2, V_DMA8 = 3, V_SKINNY = 4, V_DMA64 = 5 };

static int forced_variant()
{
    static const int v = [] {
        const char *e = getenv("FP8BS_GEMM_VARIANT");
        if (!e)
            return (int)V_AUTO;
        if (!strcmp(e, "simple"))
            return (int)V_SIMPLE;
        if (!strcmp(e, "dma"))
            return (int)V_DMA;
        if (!strcmp(e, "dma8"))
            return (int)V_DMA8;
        if (!strcmp(e, "skinny"))
            return (int)V_SKINNY;
        if (!strcmp(e, "dma64"))
            return (int)V_DMA64;
        return (int)V_AUTO;
    }();
    return v;
}

static int forced_ksplit()
{
    static const int v = [] {
        const char *e = getenv("FP8BS_GEMM_KSPLIT");
        const int n = e ? atoi(e) : 0;
        return n > 0 ? n : 0;
    }();
    return v;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GROUPED>
static hipError_t run_simple(GemmArgs a, int grid, bool out_f32, hipStream_t stream)
{
    const dim3 block(WAVES_M * WAVES_N * 64);
    if (out_f32)
        return launch(gemm_kernel<BM, BN, WAVES_M, WAVES_N, true, GROUPED>, dim3(grid), block, 0, stream, a);
    return launch(gemm_kernel<BM, BN, WAVES_M, WAVES_N, false, GROUPED>, dim3(grid), block, 0, stream, a);
}

// Persistent launch: one workgroup per CU (at most one work unit per
// workgroup when there are fewer units than CUs); the count is a multiple of
// the 8 XCDs so that the XCD-contiguous unit ranges line up with the dispatch.
constexpr int kPersistentGrid = 256;

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GROUPED, bool POW2, bool WROW = false>
static hipError_t run_dma_t(GemmArgs a, bool out_f32, hipStream_t stream)
{
    const dim3 block(WAVES_M * WAVES_N * 64);
    const int units = a.tiles_m * a.tiles_n * a.ksplit;
    const int grid = units < kPersistentGrid ? units : kPersistentGrid;
    if (GROUPED || a.ksplit == 1) {
        if (out_f32)
            return launch(gemm_dma_kernel<BM, BN, WAVES_M, WAVES_N, true, GROUPED, false, POW2, WROW>, dim3(grid),
                          block, 0, stream, a);
        return launch(gemm_dma_kernel<BM, BN, WAVES_M, WAVES_N, false, GROUPED, false, POW2, WROW>, dim3(grid), block,
                      0, stream, a);
    }
    if constexpr (!GROUPED) { // (the grouped form is never split)
        const hipError_t e = launch(gemm_dma_kernel<BM, BN, WAVES_M, WAVES_N, true, false, true, POW2, WROW>,
                                    dim3(grid), block, 0, stream, a);
        if (e != hipSuccess)
            return e;
        const int64_t MN = a.M * a.N;
        int64_t rb = (MN / 4 + 255) / 256;
        rb = rb < 4096 ? rb : 4096;
        if (out_f32)
            return launch(splitk_reduce_kernel<true>, dim3((unsigned)rb), dim3(256), 0, stream, (const float *)a.part,
                          a.y, MN, a.ksplit);
        return launch(splitk_reduce_kernel<false>, dim3((unsigned)rb), dim3(256), 0, stream, (const float *)a.part, a.y,
                      MN, a.ksplit);
    }
    return hipErrorInvalidValue;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GROUPED>
static hipError_t run_dma(GemmArgs a, bool out_f32, bool pow2, hipStream_t stream)
{
    if (pow2)
        return run_dma_t<BM, BN, WAVES_M, WAVES_N, GROUPED, true>(a, out_f32, stream);
    return run_dma_t<BM, BN, WAVES_M, WAVES_N, GROUPED, false>(a, out_f32, stream);
}

// The large-tile kernels: N a multiple of their 256-wide tile, 32-bit
// LDS-DMA offsets (256 rows of K bytes) and 32-bit store offsets (256 rows of
// N fp32).
static bool dma_ok(int64_t N, int64_t K)
{
    return N % 256 == 0 && 256 * K < ((int64_t)1 << 32) && 256 * N * 4 < ((int64_t)1 << 31);
}

// The weight-streaming kernel: at most 256 activation rows, N a multiple of
// 16, 32-bit buffer offsets (16 rows of K bytes per tile group, 128 rows of
// X), enough K blocks for the waves to share, and at most kSkinnyMaxIt of
// them per wave.
static bool skinny_ok(int64_t M, int64_t N, int64_t K)
{
    return M <= 256 && N % 16 == 0 && 128 * K < ((int64_t)1 << 31) && K / 128 >= 8 && K / 128 <= 8 * kSkinnyMaxIt;
}

// Rows up to which the weight-streaming kernel is the automatic choice (above
// them the persistent kernel, split along K where it has few tiles, is faster
// on the decode shapes).
constexpr int64_t kSkinnyMaxM = 16;

template <int TM, int TN, int D, int QX = 0>
static hipError_t run_skinny_t(GemmArgs a, bool out_f32, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.N / (TN * 16)), (unsigned)((a.M + TM * 16 - 1) / (TM * 16)));
    if (out_f32)
        return launch(gemm_skinny_kernel<TM, TN, D, true, QX>, grid, dim3(512), 0, stream, a);
    return launch(gemm_skinny_kernel<TM, TN, D, false, QX>, grid, dim3(512), 0, stream, a);
}

// The weight-streaming kernel on bf16 activations (M <= 16: one 16-row X
// tile), quantizing them itself with EXACT (QX = 1) or POW2 (QX = 2) scales,
// with the 64- or 32-row W tiles the plain kernel would pick (linear_fused
// admits no other shape).  With 64-row tiles one K block in flight per wave
// measured best (92 VGPRs, four workgroups per CU): more depth costs
// occupancy, and the other workgroups' loads hide the latency better.
template <int QX>
static hipError_t run_skinny_qx(GemmArgs a, bool out_f32, hipStream_t stream)
{
    if (a.N % 64 == 0 && a.N / 64 >= 256)
        return run_skinny_t<1, 4, 1, QX>(a, out_f32, stream);
    return run_skinny_t<1, 2, 4, QX>(a, out_f32, stream);
}

// W tile width: the widest of 64 / 32 / 16 rows that still gives at least 256
// workgroups (one per CU), so W streams from every CU; X rows per workgroup:
// the fewest 16-row tiles covering M, up to 64 rows per chunk (above that,
// each chunk of X rows re-reads W: larger chunks would re-read X from L2 once
// per 16-row W tile, which costs more).
static hipError_t run_skinny(GemmArgs a, bool out_f32, hipStream_t stream)
{
    const int64_t M = a.M, N = a.N;
    const int tn = (N % 64 == 0 && N / 64 >= 256) ? 4 : (N % 32 == 0 && N / 32 >= 256) ? 2 : 1;
    const int tm = M <= 16 ? 1 : M <= 32 ? 2 : 4;
    if (tm == 1) {
        if (tn == 4) // two K blocks in flight per wave (80 VGPRs) stream faster than four (196)
            return run_skinny_t<1, 4, 2>(a, out_f32, stream);
        if (tn == 2)
            return run_skinny_t<1, 2, 4>(a, out_f32, stream);
        return run_skinny_t<1, 1, 6>(a, out_f32, stream);
    }
    if (tm == 2) {
        if (tn == 4)
            return run_skinny_t<2, 4, 3>(a, out_f32, stream);
        if (tn == 2)
            return run_skinny_t<2, 2, 4>(a, out_f32, stream);
        return run_skinny_t<2, 1, 4>(a, out_f32, stream);
    }
    if (tn == 4)
        return run_skinny_t<4, 4, 2>(a, out_f32, stream);
    if (tn == 2)
        return run_skinny_t<4, 2, 3>(a, out_f32, stream);
    return run_skinny_t<4, 1, 4>(a, out_f32, stream);
}

// Number of K ranges for a persistent launch of `tiles` output tiles over KB
// K blocks: the split that minimizes the rounds of units per CU times the
// steps of a unit (plus a per-unit and a reduction overhead, in K-step units),
// with at least four K blocks per range.  Large products (tiles >= CUs) stay
// unsplit.
static int choose_ksplit(int64_t tiles, int64_t KB)
{
    if (tiles >= kPersistentGrid)
        return 1;
    int best = 1;
    int64_t best_cost = -1;
    for (int ks = 1; ks <= 32 && KB / ks >= 4; ++ks) {
        const int64_t rounds = (tiles * ks + kPersistentGrid - 1) / kPersistentGrid;
        const int64_t cost = rounds * ((KB + ks - 1) / ks + 2) + (ks > 1 ? 2 : 0);
        if (best_cost < 0 || cost < best_cost) {
            best_cost = cost;
            best = ks;
        }
    }
    return best;
}

enum Kind { K_SIMPLE, K_DMA128, K_DMA256, K_SKINNY, K_DMA64 };
struct Plan {
    int kind;
    int tiles_m, tiles_n, ksplit;
};

// The kernel, tiling and K split of a dense product: a function of the shape
// (and the measurement overrides) only, shared by the workspace query and
// the launch.
static Plan plan_dense(int64_t M, int64_t N, int64_t K, bool row_scaled = false)
{
    const int fv = forced_variant();
    const int64_t KB = K / BK;
    Plan p = {K_SIMPLE, (int)((M + 127) / 128), (int)(N / 128), 1};
    // weight streaming up to 16 rows; with its narrowest (16-row) W tiles only up to 8, above which
    // the persistent kernel's 64-row tiles stream the weight faster (down projection at 12 and 16
    // rows: 3% and 9%)
    const bool narrow_w = !(N % 32 == 0 && N / 32 >= 256);
    const bool stream_w = M <= (narrow_w && dma_ok(N, K) ? 8 : kSkinnyMaxM);
    if (!row_scaled && skinny_ok(M, N, K) && ((fv == V_AUTO && stream_w) || fv == V_SKINNY)) {
        p.kind = K_SKINNY;
        return p;
    }
    if (fv == V_SIMPLE || !dma_ok(N, K))
        return p;
    // 256 x 256 tiles when they fill every CU at least once, else 128 x 256; up to 128 rows
    // (decode), 64 x 256 while those tiles fit in one round of workgroups: no padding rows at
    // M = 64, and twice the units at M = 128
    const bool big = fv == V_DMA8 || (fv != V_DMA && ((M + 255) / 256) * (N / 256) >= kPersistentGrid);
    const bool rows64 =
        !big && !row_scaled &&
        ((fv == V_AUTO && M <= 128 && ((M + 63) / 64) * (N / 256) <= kPersistentGrid) || fv == V_DMA64);
    const int bm = big ? 256 : (rows64 ? 64 : 128);
    p.kind = big ? K_DMA256 : (rows64 ? K_DMA64 : K_DMA128);
    p.tiles_m = (int)((M + bm - 1) / bm);
    p.tiles_n = (int)(N / 256);
    const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
    int ks = forced_ksplit() ? forced_ksplit() : choose_ksplit(tiles, KB);
    ks = ks < (int)KB ? ks : (int)KB;
    if (row_scaled)
        ks = 1; // (its entry point takes no workspace for partial sums)
    // units are counted in int; a split product's partial sums stay addressable
    while (ks > 1 && tiles * ks > (1 << 30))
        --ks;
    p.ksplit = ks;
    return p;
}

size_t gemm_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0)
        return 0;
    const Plan p = plan_dense(M, N, K);
    return p.ksplit > 1 ? (size_t)p.ksplit * (size_t)M * (size_t)N * sizeof(float) : 0;
}

hipError_t launch_gemm(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                       int64_t K, void *y, int out_fp32, int pow2, void *workspace, hipStream_t stream)
{
    if (M == 0)
        return hipSuccess;
    GemmArgs a = {};
    a.xq = (const uint8_t *)xq;
    a.xs = xs;
    a.wq = (const uint8_t *)wq;
    a.ws = ws;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    const Plan p = plan_dense(M, N, K);
    a.tiles_m = p.tiles_m;
    a.tiles_n = p.tiles_n;
    a.ksplit = p.ksplit;
    a.part = (float *)workspace;
    switch (p.kind) {
    case K_SKINNY:
        return run_skinny(a, out_fp32 != 0, stream);
    case K_DMA256:
        return run_dma<256, 256, 4, 2, false>(a, out_fp32 != 0, pow2 != 0, stream);
    case K_DMA128:
        return run_dma<128, 256, 2, 4, false>(a, out_fp32 != 0, pow2 != 0, stream);
    case K_DMA64:
        return run_dma<64, 256, 1, 4, false>(a, out_fp32 != 0, pow2 != 0, stream);
    default:
        return run_simple<128, 128, 2, 2, false>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
    }
}

hipError_t launch_gemm_1x128(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                             int64_t K, void *y, int out_fp32, int pow2, hipStream_t stream)
{
    if (M == 0)
        return hipSuccess;
    GemmArgs a = {};
    a.xq = (const uint8_t *)xq;
    a.xs = xs;
    a.wq = (const uint8_t *)wq;
    a.ws = ws;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    const Plan p = plan_dense(M, N, K, true);
    a.tiles_m = p.tiles_m;
    a.tiles_n = p.tiles_n;
    a.ksplit = 1;
    // (POW2: the scales reach the matrix cores on the large-tile kernels; the general kernel's
    // fp32 rescale applies them as it applies any other scales)
    if (p.kind == K_DMA256)
        return pow2 ? run_dma_t<256, 256, 4, 2, false, true, true>(a, out_fp32 != 0, stream)
                    : run_dma_t<256, 256, 4, 2, false, false, true>(a, out_fp32 != 0, stream);
    if (p.kind == K_DMA128)
        return pow2 ? run_dma_t<128, 256, 2, 4, false, true, true>(a, out_fp32 != 0, stream)
                    : run_dma_t<128, 256, 2, 4, false, false, true>(a, out_fp32 != 0, stream);
    const int grid = a.tiles_m * a.tiles_n;
    const dim3 block(2 * 2 * 64);
    if (out_fp32)
        return launch(gemm_kernel<128, 128, 2, 2, true, false, true>, dim3(grid), block, 0, stream, a);
    return launch(gemm_kernel<128, 128, 2, 2, false, false, true>, dim3(grid), block, 0, stream, a);
}

// ---- the whole linear layer: bf16 activations in ---------------------------------
//
// Y = fp8_block_gemm(quant_act_1x128(X), Wq, Ws).  Decode shapes (at most 16
// rows, on shapes the weight-streaming kernel takes with W tiles of 32 or 64
// rows) run as one launch that quantizes X inside the GEMM; every other shape
// quantizes X into the workspace and runs the GEMM on it.  Either way the
// codes, scales and Y are those of the two separate calls.  (With 16-row W
// tiles the plain kernel fits two workgroups per CU and the fused one, holding
// bf16 X in flight, only one: the two calls were faster there, e.g. 25 us
// against 33 us for 1 x 14336 x 4096.)
static bool linear_fused(int64_t M, int64_t N, int64_t K)
{
    return M <= kSkinnyMaxM && skinny_ok(M, N, K) && N % 32 == 0 && N / 32 >= 256;
}

static size_t align16(size_t b) { return (b + 15) & ~(size_t)15; }

size_t linear_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || linear_fused(M, N, K))
        return 0;
    return align16((size_t)M * (size_t)K) + align16((size_t)M * (size_t)(K / BK) * sizeof(float)) +
           gemm_workspace_size(M, N, K);
}

hipError_t launch_linear(const void *x, const void *wq, const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                         int out_fp32, int pow2, void *workspace, hipStream_t stream)
{
    if (M == 0)
        return hipSuccess;
    if (linear_fused(M, N, K)) {
        GemmArgs a = {};
        a.xq = (const uint8_t *)x; // bf16 activations
        a.wq = (const uint8_t *)wq;
        a.ws = ws;
        a.y = y;
        a.M = M;
        a.N = N;
        a.K = K;
        return pow2 ? run_skinny_qx<2>(a, out_fp32 != 0, stream) : run_skinny_qx<1>(a, out_fp32 != 0, stream);
    }
    uint8_t *xq = (uint8_t *)workspace;
    float *xs = (float *)(xq + align16((size_t)M * (size_t)K));
    void *gws = (uint8_t *)xs + align16((size_t)M * (size_t)(K / BK) * sizeof(float));
    const hipError_t e = launch_quant_act(x, M, K, xq, xs, pow2 ? SCALE_POW2 : SCALE_EXACT, stream);
    if (e != hipSuccess)
        return e;
    return launch_gemm(xq, xs, wq, ws, M, N, K, y, out_fp32, pow2, gws, stream);
}

// ---- the GEMM whose epilogue quantizes its output (next layer's FP8 input) ----
//
// Fused where the dense plan is the unsplit 256 x 256 persistent kernel (each
// wave then holds whole 128-column blocks of its rows); elsewhere the GEMM
// writes bf16 Y (the caller's, or the workspace's when the caller wants none)
// and the activation quantizer reads it back.
static bool gemm_quant_fused(int64_t M, int64_t N, int64_t K)
{
    const Plan p = plan_dense(M, N, K);
    return p.kind == K_DMA256 && p.ksplit == 1;
}

size_t gemm_quant_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || gemm_quant_fused(M, N, K))
        return 0;
    return align16((size_t)M * (size_t)N * 2) + gemm_workspace_size(M, N, K);
}

hipError_t launch_gemm_quant(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                             int64_t K, void *y, void *yq, float *ys, int mode, void *workspace, hipStream_t stream)
{
    if (M == 0)
        return hipSuccess;
    const bool pow2 = mode == SCALE_POW2;
    if (gemm_quant_fused(M, N, K)) {
        GemmArgs a = {};
        a.xq = (const uint8_t *)xq;
        a.xs = xs;
        a.wq = (const uint8_t *)wq;
        a.ws = ws;
        a.y = y;
        a.yq = (uint8_t *)yq;
        a.ys = ys;
        a.M = M;
        a.N = N;
        a.K = K;
        const Plan p = plan_dense(M, N, K);
        a.tiles_m = p.tiles_m;
        a.tiles_n = p.tiles_n;
        a.ksplit = 1;
        const int units = a.tiles_m * a.tiles_n;
        const int grid = units < kPersistentGrid ? units : kPersistentGrid;
        if (pow2)
            return launch(gemm_dma_kernel<256, 256, 4, 2, false, false, false, true, false, 2>, dim3(grid),
                          dim3(512), 0, stream, a);
        return launch(gemm_dma_kernel<256, 256, 4, 2, false, false, false, false, false, 1>, dim3(grid), dim3(512),
                      0, stream, a);
    }
    void *yb = y != nullptr ? y : workspace;
    void *gws = (uint8_t *)workspace + align16((size_t)M * (size_t)N * 2);
    // the kernel fp8_block_gemm itself would run (one row: the GEMV), so that Y is its Y
    const hipError_t e = gemv_ok(M, N, K) ? launch_gemv(xq, xs, wq, ws, N, K, yb, 0, 0, stream)
                                          : launch_gemm(xq, xs, wq, ws, M, N, K, yb, 0, pow2 ? 1 : 0, gws, stream);
    if (e != hipSuccess)
        return e;
    return launch_quant_act(yb, M, N, yq, ys, mode, stream);
}

// Grouped workspace: the two tile counts, padded to 16 bytes, then table A
// (256-row tiles: ceil(M_total / 256) + E entries) and table B (the experts'
// last tiles of at most 128 rows: E entries).  Forced to 128-row tiles
// (FP8BS_GEMM_VARIANT=dma), table A holds every tile and B stays empty.
constexpr size_t kGroupHeader = 16;

static bool grouped_small_tiles() { return forced_variant() == V_DMA; }

static int64_t grouped_cap_a(int64_t E, int64_t M_total)
{
    const int64_t bm = grouped_small_tiles() ? 128 : 256;
    return (M_total + bm - 1) / bm + E;
}

size_t grouped_workspace_size(int64_t E, int64_t M_total, int64_t N, int64_t K)
{
    if (E <= 0 || M_total <= 0 || forced_variant() == V_SIMPLE || !dma_ok(N, K))
        return 0;
    return kGroupHeader + (size_t)(grouped_cap_a(E, M_total) + E) * sizeof(GroupTile);
}

hipError_t launch_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void *y,
                               int out_fp32, int pow2, void *workspace, hipStream_t stream)
{
    if (M_total == 0)
        return hipSuccess;
    GemmArgs a = {};
    a.xq = (const uint8_t *)xq;
    a.xs = xs;
    a.wq = (const uint8_t *)wq;
    a.ws = ws;
    a.offsets = offsets;
    a.y = y;
    a.M = M_total;
    a.N = N;
    a.K = K;
    a.E = E;
    a.ksplit = 1;
    if (grouped_workspace_size(E, M_total, N, K) > 0) {
        const int cap_a = (int)grouped_cap_a(E, M_total), cap_b = (int)E;
        int32_t *count = (int32_t *)workspace;
        GroupTile *tab_a = (GroupTile *)((uint8_t *)workspace + kGroupHeader);
        GroupTile *tab_b = tab_a + cap_a;
        a.tiles_n = (int)(N / 256);
        if (grouped_small_tiles()) {
            hipError_t e = launch(grouped_tile_table_kernel<128, 0>, dim3(1), dim3(64), 0, stream, offsets, E, M_total,
                                  cap_a, tab_a, cap_b, tab_b, count);
            if (e != hipSuccess)
                return e;
            a.tiles_m = cap_a;
            a.gtab = tab_a;
            a.gcount = count;
            return run_dma<128, 256, 2, 4, true>(a, out_fp32 != 0, pow2 != 0, stream);
        }
        hipError_t e = launch(grouped_tile_table_kernel<256, 128>, dim3(1), dim3(64), 0, stream, offsets, E, M_total,
                              cap_a, tab_a, cap_b, tab_b, count);
        if (e != hipSuccess)
            return e;
        // 256-row tiles first, then the experts' short last tiles with 128-row tiles
        a.tiles_m = cap_a;
        a.gtab = tab_a;
        a.gcount = count;
        if ((e = run_dma<256, 256, 4, 2, true>(a, out_fp32 != 0, pow2 != 0, stream)) != hipSuccess)
            return e;
        a.tiles_m = cap_b;
        a.gtab = tab_b;
        a.gcount = count + 1;
        return run_dma<128, 256, 2, 4, true>(a, out_fp32 != 0, pow2 != 0, stream);
    }
    a.tiles_m = (int)((M_total + 127) / 128 + E);
    a.tiles_n = (int)(N / 128);
    return run_simple<128, 128, 2, 2, true>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
}

// ---- the grouped GEMM's row-tile tables without a caller workspace ----------
// For callers that cannot allocate (graph capture, serving loops): the tables
// live in this file-scope device array, one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is handed to kernels.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kScratchDevices];
} // namespace

hipError_t noalloc_scratch(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess)
            return e;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

} // namespace fp8bs
