// fp8bs_gemm.hip -- block-scaled FP8 GEMM and its grouped (MoE) form, gfx950.
//
// The article "NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
// precision training", section "Technical breakthrough": linear layers run FP8
// math on operands quantized per 1x128 (activations) and 128x128 (weights)
// block.  Here
//   Y[m, n] = sum_kb (xs[m, kb] * ws[n/128, kb]) * P[m, n, kb],
//   P[m, n, kb] = sum_{k in kb} decode(xq[m, k]) * decode(wq[n, k]),
// with P from the CDNA4 FP8 matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4,
// hardware block scales neutral) into a fresh fp32 partial per 128-wide K
// block, and the fp32 scale product applied by one FMA per output element
// and K block into the running fp32 accumulator.
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
// Staging.  Global -> registers -> LDS, double-buffered, one barrier per K
// block; the next block's global loads are in flight while the current one
// is multiplied.  LDS rows are 128 bytes; the 16-byte chunk c of row r is
// stored at chunk c ^ ((r >> 1) & 7), so the 16 rows read by one 16-lane
// group spread over all banks.
//
// Workgroup order.  Consecutive workgroup ids are dispatched round-robin to
// the 8 XCDs, each with its own L2; ids are remapped so that each XCD gets a
// contiguous range of tiles, walked GROUP_M m-tiles at a time so that
// workgroups resident together share their weight and activation tiles.
#include "fp8bs_device.hpp"
#include "fp8bs_internal.hpp"

#include <stdlib.h>
#include <string.h>

namespace fp8bs {

constexpr int BK = 128;        // K block = scale block
constexpr int NUM_XCD = 8;     // MI355X: 8 accelerator complex dies
constexpr int GROUP_M = 8;

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

template <int BM, int BN, int WAVES_M, int WAVES_N, bool OUT_F32, bool GROUPED>
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
        const float sw = ws_row[kb];
        float sc[C::TM];
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            sc[i] = xs_row[i][kb] * sw;

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
                // format 0 = FP8 E4M3 for both operands; E8M0 scale 127 = 2^0 (neutral)
                const v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw[j], bx[i], v4f{0.f, 0.f, 0.f, 0.f},
                                                                               0, 0, 0, 127, 0, 127);
                acc[i][j] = __builtin_elementwise_fma(v4f{sc[i], sc[i], sc[i], sc[i]}, p, acc[i][j]);
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
// shapes (M in the thousands):
//   - large workgroup tiles (BM x BN = 256 x 256 over 8 waves, or 128 x 256
//     over 4) of 64 x 128 wave tiles, so each K block moves (BM + BN) * 128
//     bytes for 2 * BM * BN * 128 FLOP and each wave reads 24 KiB of LDS per
//     32 MFMAs.  With 8 waves each SIMD holds two, so one wave's fp32 rescale
//     (VALU) runs while the other's MFMAs keep the matrix core busy;
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
//   - STAGES LDS buffers: the loads of block kb + STAGES - 1 are in flight
//     while block kb is multiplied; one barrier per K block both publishes
//     block kb and retires the reads of the buffer the next loads refill.
//     Waits are explicit (s_waitcnt vmcnt with the count of loads issued after
//     the ones needed), with every count a compile-time constant;
//   - the weight scale of a K block is one scalar load; each wave fetches the
//     activation scales of its own 64 rows (one dword per lane) with its
//     operands, into a region of the stage that only it reads.
template <int BM, int BN, int WAVES_M, int WAVES_N, int STAGES_>
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
    static constexpr int DPW = XG + WG + 1; // LDS-DMA instructions per wave per stage (+1: scales)
    static_assert(STAGES == 2 || STAGES == 3, "two or three LDS stages");
    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "row groups must split evenly over the waves");
    static_assert(BM % 16 == 0, "16-row layout groups must not straddle X and W");
    static_assert(WM == 64, "one activation-scale dword per lane covers the wave's 64 rows");
    static_assert(WN % 16 == 0, "wave tile must be made of 16x16 MFMA tiles");
    static_assert(WN <= 128 && 128 % WN == 0, "a wave's columns must lie in one 128-wide weight scale block");
    static_assert(STAGES * STAGE_BYTES <= 160 * 1024, "LDS budget of a gfx950 CU");
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

// s_waitcnt lgkmcnt(0) with vmcnt / expcnt left alone.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Raw buffer resource over [base, base + bytes) (gfx9 descriptor word 3:
// 32-bit data format, no swizzle); loads past `bytes` return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes >= 0xffffffffLL ? (int)0xffffffffu : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// Geometry of one output tile of the persistent kernels.
struct TileGeo {
    int64_t row_begin, row_end; // rows of X / Y: [row_begin, row_end)
    int64_t n0;                 // first column of Y (row of W)
    const uint8_t *wq;          // this tile's weight matrix (the expert's, for the grouped form)
    const float *ws;
};

// Tile of virtual id v (< tiles_m * tiles_n), or false for a grouped tile
// past the last row tile of its expert list.
template <int BM, int BN, bool GROUPED>
__device__ __forceinline__ bool tile_geo(const GemmArgs &a, int v, int ntiles, TileGeo &g)
{
    int tm, tn;
    tile_of(v, ntiles, a.tiles_m, a.tiles_n, tm, tn);
    g.wq = a.wq;
    g.ws = a.ws;
    if (GROUPED) {
        int e;
        if (!expert_of_tile<BM>(a.offsets, a.E, a.M, tm, e, g.row_begin, g.row_end))
            return false;
        g.wq += (int64_t)e * a.N * a.K;
        g.ws += (int64_t)e * (a.N / 128) * (a.K / BK);
    } else {
        g.row_begin = (int64_t)tm * BM;
        g.row_end = (g.row_begin + BM) < a.M ? (g.row_begin + BM) : a.M;
    }
    g.n0 = (int64_t)tn * BN;
    return true;
}

// Persistent form: gridDim.x workgroups (one per CU) walk the virtual tiles
// v = blockIdx.x, blockIdx.x + gridDim.x, ...  All (tile, K block) steps of
// a workgroup form one stream through the two LDS stages: the operands of
// step s + 2 are issued in the middle of step s, as soon as every wave has
// finished reading the stage they refill (a full step of lookahead), and the
// fragments of step s + 1 are read into registers during the last MFMA
// groups of step s, so the matrix cores never wait on LDS at a step
// boundary; a tile's output stores drain while the next tile computes.  Stores are buffer stores
// whose out-of-range rows the hardware drops.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool OUT_F32, bool GROUPED>
__global__ __launch_bounds__(WAVES_M *WAVES_N * 64) void gemm_dma_kernel(GemmArgs a)
{
    using C = DmaCfg<BM, BN, WAVES_M, WAVES_N, 2>;
    __shared__ __attribute__((aligned(1024))) uint8_t lds[C::STAGES * C::STAGE_BYTES];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    const int64_t K = a.K, KB = K / BK, N = a.N;
    const int ntiles = a.tiles_m * a.tiles_n;
    const int sub = lane >> 3, slot = lane & 7;
    const int fr = lane & 15, fg = lane >> 4;

    // ---- DMA cursor: the tile and K block whose operands load next ----
    int dv = blockIdx.x;
    TileGeo dt;
    bool dvalid = false;
    while (dv < ntiles && !(dvalid = tile_geo<BM, BN, GROUPED>(a, dv, ntiles, dt)))
        dv += gridDim.x;
    if (!dvalid)
        return; // no tile for this workgroup (uniform)
    TileGeo ct = dt; // tile of the step being computed
    int64_t dkb = 0;

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
    // (the resources are rebuilt per issue from the tile's bases and row
    // count: the host pass of this compiler emits no launch stub for a kernel
    // holding an array of buffer resources)
    const uint8_t *xbase, *wbase;
    const float *sbase;
    int64_t xrows;
    const int r0 = tile_row(wave * 8 + sub);
    const uint32_t loff = (uint32_t)(r0 * K) + (uint32_t)((slot ^ (r0 & 7)) << 4);
    const uint32_t soff = (uint32_t)((wm * C::WM + lane) * KB * 4);
    auto dma_setup = [&](const TileGeo &g) {
        xbase = a.xq + g.row_begin * K;
        xrows = g.row_end - g.row_begin;
        wbase = g.wq + g.n0 * K;
        sbase = a.xs + g.row_begin * KB;
    };
    // Loads of K block kb into `stage`.  With live == false every range is
    // empty, so the same instructions move nothing (the hardware range check
    // drops them): the caller issues them unconditionally, keeping the MFMA
    // stream they sit in free of branches.
    auto issue = [&](int64_t kb, int stage, bool live = true) {
        uint8_t *L = lds + stage * C::STAGE_BYTES;
        const int ko = (int)(kb * BK);
        const int64_t rows = live ? xrows : 0;
#pragma unroll
        for (int t = 0; t < C::XG; ++t) {
            const int64_t left = rows - (int64_t)GROW * t;
            const __amdgpu_buffer_rsrc_t xr = make_rsrc(xbase + (int64_t)GROW * t * K, left > 0 ? left * K : 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (LDS_AS void *)(L + (wave + C::NW * t) * 1024), 16,
                                                     (int)loff, ko, 0, 0);
        }
        const __amdgpu_buffer_rsrc_t wl = make_rsrc(wbase, live ? (int64_t)BN * K : 0);
#pragma unroll
        for (int t = 0; t < C::WG; ++t)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(wl, (LDS_AS void *)(L + BM * BK + (wave + C::NW * t) * 1024),
                                                     16, (int)loff, ko + (int)(GROW * t * K), 0, 0);
        const __amdgpu_buffer_rsrc_t sl = make_rsrc(sbase, rows * KB * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sl, (LDS_AS void *)(L + C::XS_OFF + wave * 256), 4, (int)soff,
                                                 (int)(kb * 4), 0, 0);
    };
    // advance the DMA cursor by one K block; false at the end of the stream
    auto dma_next = [&]() {
        if (++dkb < KB)
            return true;
        dkb = 0;
        do {
            dv += gridDim.x;
        } while (dv < ntiles && !tile_geo<BM, BN, GROUPED>(a, dv, ntiles, dt));
        if (dv >= ntiles)
            return false;
        dma_setup(dt);
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
    // previous step's last two MFMA groups run.  W fragments rotate through
    // a ring of three (the group being multiplied and the next two).
    v8i bx[C::TM];
    v8i awq[3];
    float sc[C::TM];
    auto ws_of = [&](const TileGeo &g) {
        return (const CONST_AS float *)(g.ws + ((g.n0 + wn * C::WN) / 128) * KB);
    };
    auto sync = [&]() {
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    auto rescale = [&](int t, const v4f &p) {
        const int i = t % C::TM, j = t / C::TM;
        acc[i][j] = __builtin_elementwise_fma(v4f{sc[i], sc[i], sc[i], sc[i]}, p, acc[i][j]);
    };
    static_assert(C::TN >= 4, "the W-fragment ring needs at least four groups per step");

    // One K block from registers.  Group j (TM MFMAs on one W fragment)
    // reads the W fragment of group j + 2, so each LDS read has two groups of
    // MFMAs to land.  The rescale of MFMA tile t is issued after the MFMA of
    // tile t + 1, so the matrix core has the next product queued while the
    // VALU applies the previous one.  Before group TN - 2 every wave waits for
    // the next step's operands (the most recent loads it issued) and for its
    // own LDS reads (the last read of this stage was issued in group TN - 3),
    // and passes the barrier: the next stage is then complete for all waves
    // and no wave reads this stage any more, so the loads issued at the top of
    // the next step may refill it.  Groups TN - 2 and TN - 1 then read the
    // next step's first two W fragments and scales, and each MFMA of the last
    // group frees its X fragment registers for the next step's.  (For the last
    // step of a workgroup those reads fetch data that is never used; the
    // barrier is uniform.)
    auto compute = [&](int stage, float sw_next, auto &&after_barrier) __attribute__((always_inline)) {
        const uint8_t *L = lds + stage * C::STAGE_BYTES;
        const uint8_t *Ln = lds + (stage ^ 1) * C::STAGE_BYTES;
        v4f part[2];
        float xs_next[C::TM];
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
            const bool last = j + 1 == C::TN;
            if (j + 2 < C::TN) {
                awq[(j + 2) % 3] = frag(L + wo[0] + (j + 2) * 2048, L + wo[1] + (j + 2) * 2048);
            } else if (j + 2 == C::TN) {
                wait_vmcnt<0>();
                wait_lgkmcnt0();
                sync();
                after_barrier();
                awq[(j + 2) % 3] = frag(Ln + wo[0], Ln + wo[1]);
#pragma unroll
                for (int i = 0; i < C::TM; ++i)
                    xs_next[i] = *(const float *)(Ln + so + i * 64);
            } else {
                awq[(j + 2) % 3] = frag(Ln + wo[0] + 2048, Ln + wo[1] + 2048);
            }
            // the reads above stay ahead of this group's MFMAs (the machine
            // scheduler would otherwise sink them to where the registers they
            // fill are next used, shrinking the prefetch distance to zero)
            __builtin_amdgcn_sched_barrier(0);
            const v8i aw = awq[j % 3];
#pragma unroll
            for (int i = 0; i < C::TM; ++i) {
                const int t = j * C::TM + i;
                part[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(aw, bx[i], v4f{0.f, 0.f, 0.f, 0.f},
                                                                               0, 0, 0, 127, 0, 127);
                if (t > 0)
                    rescale(t - 1, part[(t - 1) & 1]);
                if (last)
                    bx[i] = frag(Ln + xo[0] + i * 2048, Ln + xo[1] + i * 2048);
            }
            // issue order: each MFMA followed by the previous rescale (and in
            // the last group by the next step's X fragment it freed)
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
            for (int i = 1; i < C::TM; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (last)
                    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
            }
            if (last)
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        rescale(C::TM * C::TN - 1, part[(C::TM * C::TN - 1) & 1]);
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            sc[i] = xs_next[i] * sw_next;
        // the next step's groups 0 and 1 were read into slots TN % 3 and
        // (TN + 1) % 3; move them to slots 0 and 1
        const v8i n0 = awq[C::TN % 3], n1 = awq[(C::TN + 1) % 3];
        awq[0] = n0;
        awq[1] = n1;
    };

    // Output of a finished tile: buffer stores over the tile's own rows, so
    // rows past row_end are dropped by the range check, not by a branch.
    auto epilogue = [&](const TileGeo &g) {
        constexpr int ES = OUT_F32 ? 4 : 2;
        const __amdgpu_buffer_rsrc_t yr =
            make_rsrc((const uint8_t *)a.y + (g.row_begin * N + g.n0) * ES, (g.row_end - g.row_begin) * N * ES);
#pragma unroll
        for (int i = 0; i < C::TM; ++i) {
            const int m = wm * C::WM + i * 16 + fr;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
                const int n = wn * C::WN + j * 16 + fg * 4;
                const int off = (int)(((int64_t)m * N + n) * ES);
                const v4f v = acc[i][j];
                if (OUT_F32) {
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), yr, off, 0, 0);
                } else {
                    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
                    const bf2 p0 = __builtin_convertvector(__builtin_shufflevector(v, v, 0, 1), bf2);
                    const bf2 p1 = __builtin_convertvector(__builtin_shufflevector(v, v, 2, 3), bf2);
                    __builtin_amdgcn_raw_buffer_store_b64(
                        u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)}, yr, off, 0, 0);
                }
                acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
            }
        }
    };

    // prologue: the first step's operands, fragments and scales
    dma_setup(dt);
    issue(0, 0);
    bool dmore = dma_next();
    wait_vmcnt<0>();
    sync();
    {
        const float sw = ws_of(ct)[0];
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            sc[i] = *(const float *)(lds + so + i * 64) * sw;
#pragma unroll
        for (int i = 0; i < C::TM; ++i)
            bx[i] = frag(lds + xo[0] + i * 2048, lds + xo[1] + i * 2048);
        awq[0] = frag(lds + wo[0], lds + wo[1]);
        awq[1] = frag(lds + wo[0] + 2048, lds + wo[1] + 2048);
    }

    // Lookahead: the operands of step s + 1 are in flight (or landed) while
    // step s is computed; those of step s + 2 are issued right after the
    // barrier in the middle of step s, the earliest point at which every wave
    // has finished reading the stage they refill.  Per lookahead step only a
    // flag and the address of its weight scale are carried; the tile of the
    // step being computed advances with its own cursor.
    int cv = dv;
    bool has1 = dmore;
    const CONST_AS float *wsp1 = ws_of(ct);
    if (has1) {
        wsp1 = ws_of(dt) + dkb;
        issue(dkb, 1);
        dmore = dma_next();
    }

    int stage = 0;
    int64_t ckb = 0;
    bool advance = false; // the cursor's step was issued during the previous step
    while (true) {
        if (advance)
            dmore = dma_next();
        float sw_next = 0.f;
        if (has1) {
            sw_next = *wsp1;
            // Take the scalar load's result right away: loads through the
            // scalar cache may return out of order, so while one is
            // outstanding every wait for an LDS read has to be lgkmcnt(0),
            // which would also wait for the fragment reads issued ahead.
            asm volatile("" ::"s"(sw_next));
        }
        const bool has2 = dmore;
        const int64_t kb2 = dkb;
        const CONST_AS float *wsp2 = has2 ? ws_of(dt) + dkb : wsp1;
        // only the loads go in the middle of the MFMA stream; the cursor
        // advances (and sets up the next tile's loads) at the top of the
        // next step
        compute(stage, sw_next, [&]() { issue(kb2, stage, has2); });
        advance = has2;
        stage ^= 1;
        if (++ckb == KB) {
            epilogue(ct);
            ckb = 0;
            if (has1) {
                do {
                    cv += gridDim.x;
                } while (!tile_geo<BM, BN, GROUPED>(a, cv, ntiles, ct));
            }
        }
        if (!has1)
            break;
        has1 = has2;
        wsp1 = wsp2;
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
template <int TM, int TN, int D, bool OUT_F32>
__global__ __launch_bounds__(512) void gemm_skinny_kernel(GemmArgs a)
{
    constexpr int NW = 8;
    constexpr int LPB = 2 * TN + 3 * TM; // loads per K block: W lo/hi, X lo/hi, X scale
    static_assert((D - 1) * LPB < 64, "outstanding loads must fit the vmcnt field");
    __shared__ __attribute__((aligned(16))) float red[NW][TM * 16][TN * 16];

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
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.xq + m0 * K, mrows * K);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.xs + m0 * KB, mrows * KB * 4);
    const __amdgpu_buffer_rsrc_t none = make_rsrc(a.xq, 0);
    const int loff = (int)(fr * K + fg * 32);
    const int soff = (int)(fr * KB * 4);
    const CONST_AS float *ws_row = (const CONST_AS float *)(a.ws + (n0 / 128) * KB);

    const int nk = wave < KB ? (int)((KB - wave + NW - 1) / NW) : 0; // this wave's K blocks

    v8i wf[D][TN], xf[D][TM];
    float xv[D][TM];
    // Loads of this wave's it-th K block into ring slot `slot`.  Blocks past
    // the end issue the same instructions on an empty range (no traffic), so
    // every step issues LPB loads and the waits below are fixed counts.
    auto load = [&](int slot, int it) {
        const bool live = it < nk;
        const int kb = live ? (int)(wave + (int64_t)it * NW) : 0;
        const __amdgpu_buffer_rsrc_t w_ = live ? wr : none, x_ = live ? xr : none, s_ = live ? sr : none;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            const int so = kb * BK + (int)(j * 16 * K);
            const u32x4 lo = __builtin_amdgcn_raw_buffer_load_b128(w_, loff, so, 0);
            const u32x4 hi = __builtin_amdgcn_raw_buffer_load_b128(w_, loff + 16, so, 0);
            wf[slot][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        // (the X row of a lane is in the per-lane offset, so a row past M
        // is out of range however the hardware counts the scalar offset)
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

#pragma unroll
    for (int d = 0; d < D; ++d)
        load(d, d);
    for (int base = 0; base < nk; base += D) {
#pragma unroll
        for (int d = 0; d < D; ++d) {
            const int it = base + d;
            wait_vmcnt<(D - 1) * LPB>(); // block `it` landed; D - 1 younger blocks may fly
            if (it < nk) {
                const float sw = ws_row[wave + (int64_t)it * NW];
                float sc[TM];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    sc[i] = xv[d][i] * sw;
                v4f part[2];
#pragma unroll
                for (int t = 0; t < TM * TN; ++t) {
                    const int i = t % TM, j = t / TM;
                    part[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf[d][j], xf[d][i],
                                                                                   v4f{0.f, 0.f, 0.f, 0.f}, 0, 0,
                                                                                   0, 127, 0, 127);
                    if (t > 0) {
                        const int pi = (t - 1) % TM, pj = (t - 1) / TM;
                        acc[pi][pj] = __builtin_elementwise_fma(v4f{sc[pi], sc[pi], sc[pi], sc[pi]},
                                                                part[(t - 1) & 1], acc[pi][pj]);
                    }
                }
                constexpr int T = TM * TN;
                acc[TM - 1][TN - 1] = __builtin_elementwise_fma(v4f{sc[TM - 1], sc[TM - 1], sc[TM - 1], sc[TM - 1]},
                                                                part[(T - 1) & 1], acc[TM - 1][TN - 1]);
            }
            load(d, it + D);
        }
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

// ---- variant table -----------------------------------------------------------------
//
// A shape picks its kernel from (M, N, K) alone -- never from out_dtype -- so
// the fp32 and bf16 outputs of one shape come from the same arithmetic.
// FP8BS_GEMM_VARIANT=simple|dma (read once) forces a kernel where its shape
// constraints allow, for measurements.

enum Variant { V_AUTO = 0, V_SIMPLE = 1, V_DMA = 2, V_DMA8 = 3 };
// (V_AUTO also picks the weight-streaming kernel for few rows)

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
        return (int)V_AUTO;
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

// Persistent launch: one workgroup per CU (at most one tile per workgroup
// when there are fewer tiles than CUs); the count is a multiple of the 8
// XCDs so that tile_of's XCD-contiguous ranges line up with the dispatch.
constexpr int kPersistentGrid = 256;

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GROUPED>
static hipError_t run_dma(GemmArgs a, int ntiles, bool out_f32, hipStream_t stream)
{
    const dim3 block(WAVES_M * WAVES_N * 64);
    const int grid = ntiles < kPersistentGrid ? ntiles : kPersistentGrid;
    if (out_f32)
        return launch(gemm_dma_kernel<BM, BN, WAVES_M, WAVES_N, true, GROUPED>, dim3(grid), block, 0, stream, a);
    return launch(gemm_dma_kernel<BM, BN, WAVES_M, WAVES_N, false, GROUPED>, dim3(grid), block, 0, stream, a);
}

// The large-tile kernels: N a multiple of their 256-wide tile, 32-bit
// LDS-DMA offsets (256 rows of K bytes) and 32-bit store offsets (256 rows of
// N fp32), and enough rows for 128-row tiles to be worth it.
static bool dma_ok(int64_t rows, int64_t N, int64_t K)
{
    return N % 256 == 0 && 256 * K < ((int64_t)1 << 32) && 256 * N * 4 < ((int64_t)1 << 31) && rows >= 128;
}

// The weight-streaming kernel: at most 128 activation rows, N a multiple of
// 16, 32-bit buffer offsets (16 rows of K bytes per tile group, 128 rows of
// X), and enough K blocks for the waves to share.
static bool skinny_ok(int64_t M, int64_t N, int64_t K)
{
    return M <= 256 && N % 16 == 0 && 128 * K < ((int64_t)1 << 31) && K / 128 >= 8;
}

template <int TM, int TN, int D>
static hipError_t run_skinny_t(GemmArgs a, bool out_f32, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.N / (TN * 16)), (unsigned)((a.M + TM * 16 - 1) / (TM * 16)));
    if (out_f32)
        return launch(gemm_skinny_kernel<TM, TN, D, true>, grid, dim3(512), 0, stream, a);
    return launch(gemm_skinny_kernel<TM, TN, D, false>, grid, dim3(512), 0, stream, a);
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
        if (tn == 4)
            return run_skinny_t<1, 4, 4>(a, out_f32, stream);
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

size_t gemm_workspace_size(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                       int64_t K, void *y, int out_fp32, void *, hipStream_t stream)
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
    const int fv = forced_variant();
    if (fv == V_AUTO && skinny_ok(M, N, K))
        return run_skinny(a, out_fp32 != 0, stream);
    if (fv != V_SIMPLE && fv != V_DMA && dma_ok(M, N, K) && M >= 256) {
        a.tiles_m = (int)((M + 255) / 256);
        a.tiles_n = (int)(N / 256);
        return run_dma<256, 256, 4, 2, false>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
    }
    if (fv != V_SIMPLE && dma_ok(M, N, K)) {
        a.tiles_m = (int)((M + 127) / 128);
        a.tiles_n = (int)(N / 256);
        return run_dma<128, 256, 2, 4, false>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
    }
    a.tiles_m = (int)((M + 127) / 128);
    a.tiles_n = (int)(N / 128);
    return run_simple<128, 128, 2, 2, false>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
}

hipError_t launch_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void *y,
                               int out_fp32, hipStream_t stream)
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
    const int fv = forced_variant();
    if (fv != V_SIMPLE && fv != V_DMA && dma_ok(M_total, N, K)) {
        a.tiles_m = (int)((M_total + 255) / 256 + E);
        a.tiles_n = (int)(N / 256);
        return run_dma<256, 256, 4, 2, true>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
    }
    a.tiles_m = (int)((M_total + 127) / 128 + E);
    if (fv != V_SIMPLE && dma_ok(M_total, N, K)) {
        a.tiles_n = (int)(N / 256);
        return run_dma<128, 256, 2, 4, true>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
    }
    a.tiles_n = (int)(N / 128);
    return run_simple<128, 128, 2, 2, true>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
}

} // namespace fp8bs
