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

// ---- variant table -----------------------------------------------------------------

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GROUPED>
static hipError_t run(GemmArgs a, int grid, bool out_f32, hipStream_t stream)
{
    const dim3 block(WAVES_M * WAVES_N * 64);
    if (out_f32)
        return launch(gemm_kernel<BM, BN, WAVES_M, WAVES_N, true, GROUPED>, dim3(grid), block, 0, stream, a);
    return launch(gemm_kernel<BM, BN, WAVES_M, WAVES_N, false, GROUPED>, dim3(grid), block, 0, stream, a);
}

size_t gemm_workspace_size(int64_t, int64_t, int64_t) { return 0; }

hipError_t launch_gemm(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                       int64_t K, void *y, int out_fp32, void *, hipStream_t stream)
{
    if (M == 0)
        return hipSuccess;
    constexpr int BM = 128, BN = 128;
    GemmArgs a = {};
    a.xq = (const uint8_t *)xq;
    a.xs = xs;
    a.wq = (const uint8_t *)wq;
    a.ws = ws;
    a.y = y;
    a.M = M;
    a.N = N;
    a.K = K;
    a.tiles_m = (int)((M + BM - 1) / BM);
    a.tiles_n = (int)(N / BN);
    return run<BM, BN, 2, 2, false>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
}

hipError_t launch_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void *y,
                               int out_fp32, hipStream_t stream)
{
    if (M_total == 0)
        return hipSuccess;
    constexpr int BM = 128, BN = 128;
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
    a.tiles_m = (int)((M_total + BM - 1) / BM + E);
    a.tiles_n = (int)(N / BN);
    return run<BM, BN, 2, 2, true>(a, a.tiles_m * a.tiles_n, out_fp32 != 0, stream);
}

} // namespace fp8bs
