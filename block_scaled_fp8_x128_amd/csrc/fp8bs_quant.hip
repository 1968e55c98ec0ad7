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
            // (default cache policy: the codes are the next GEMM's operand, which
            // then reads them from the caches; the recalibration's quantizer,
            // whose gigabytes of output would only evict, streams them instead)
            q[b * 16 + c] = codes;
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
// A workgroup of 256 BW threads quantizes BW horizontally adjacent 128x128
// blocks of one 128-row band (BW = 4 for a tensor with a multiple of 4 K
// blocks, else 2 for a multiple of 2, else 1).  Lane l of a wave reads the 16-byte
// chunk l % (16 BW) of row l / (16 BW) of a group of rows, so one load
// instruction covers 256 BW contiguous bytes of each of 4 / BW rows; thread t
// covers its row and the rows 16, 32, ..., 112 below it: eight loads in flight
// per thread, the whole band held in registers across the amax reduction, so
// the bf16 input is read from HBM exactly once.  Against one block per
// workgroup (four 256-byte row pieces per instruction), four blocks measured
// 7% faster (65.8% -> 70.7% of HBM peak over 32 weights of the 8B layer
// shapes).  A launch covers up to QW_MAX_TENSORS tensors; workgroup ids are
// concatenated over the tensors' band grids.
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

template <int MODE, int BW>
__global__ __launch_bounds__(QW_THREADS * BW) void quant_w_kernel(QWArgs a)
{
    constexpr int NWV = 4 * BW, CPR = 16 * BW, RPI = 4 / BW; // waves; chunks per band row; rows per instruction
    __shared__ uint32_t red[NWV][BW];
    const int64_t tile = blockIdx.x;
    int i = 0;
    while (i + 1 < a.count && tile >= a.tile_begin[i + 1])
        ++i;
    const int64_t K = a.K[i];
    const int64_t KB = K / 128, KP = (KB + BW - 1) / BW; // K blocks; groups of BW of them
    const int64_t local = tile - a.tile_begin[i];
    const int64_t nb = local / KP, kp = local % KP;

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int c = lane % CPR, blk = c >> 4; // chunk within the band row, and its block
    const int64_t kb = BW * kp + blk;
    const bool on = kb < KB; // (a partial last group when BW does not divide KB)
    const int r0 = RPI * wave + lane / CPR; // 0 .. 15
    const int64_t base = (nb * 128 + r0) * K + kp * 128 * BW + c * 8; // element offset of the first chunk
    const int64_t rstep = 16 * K;                                     // 16 rows
    const uint16_t *w = a.w[i];

    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = on ? __builtin_nontemporal_load((const u32x4 *)(w + base + j * rstep)) : u32x4{0u, 0u, 0u, 0u};

    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t cm = chunk_max_mag(v[j]);
        m = m > cm ? m : cm;
    }
    m = row16_max(m); // DPP row d (lanes 16 d .. 16 d + 15) holds block d % BW
    {
        uint32_t r[4];
#pragma unroll
        for (int d = 0; d < 4; ++d)
            r[d] = __builtin_amdgcn_readlane(m, 16 * d);
        if (lane == 0) {
#pragma unroll
            for (int h = 0; h < BW; ++h) {
                uint32_t x = 0;
#pragma unroll
                for (int d = h; d < 4; d += BW)
                    x = x > r[d] ? x : r[d];
                red[wave][h] = x;
            }
        }
    }
    __syncthreads();
    uint32_t bm = red[0][blk];
#pragma unroll
    for (int j = 1; j < NWV; ++j)
        bm = bm > red[j][blk] ? bm : red[j][blk];

    BlockQuant<MODE> bq;
    bq.init(amax_value(bm));
    if (on) {
        uint8_t *q = a.q[i];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const u32x2 codes = quant_chunk<MODE>(v[j], bq);
            __builtin_nontemporal_store(codes, (u32x2 *)(q + base + j * rstep));
        }
        if (t < CPR && (t & 15) == 0) // lane 16 h of wave 0 writes block h's scale
            a.s[i][nb * KB + kb] = bq.s;
    }
}

template <int BW>
static hipError_t launch_quant_w_bw(const WTensor *t, int64_t n, int mode, hipStream_t stream)
{
    QWArgs a = {};
    int64_t tiles = 0;
    for (int64_t j = 0; j < n; ++j) {
        const WTensor &wt = t[j];
        a.tile_begin[j] = tiles;
        a.w[j] = (const uint16_t *)wt.w;
        a.q[j] = (uint8_t *)wt.q;
        a.s[j] = wt.s;
        a.K[j] = wt.K;
        tiles += (wt.N / 128) * ((wt.K / 128 + BW - 1) / BW);
    }
    a.tile_begin[n] = tiles;
    a.count = (int)n;
    if (tiles == 0)
        return hipSuccess;
    if (mode == SCALE_POW2)
        return launch(quant_w_kernel<SCALE_POW2, BW>, dim3((unsigned)tiles), dim3(QW_THREADS * BW), 0, stream, a);
    return launch(quant_w_kernel<SCALE_EXACT, BW>, dim3((unsigned)tiles), dim3(QW_THREADS * BW), 0, stream, a);
}

// Each tensor goes to the widest band that divides its K blocks: one launch
// per band width present, each over up to QW_MAX_TENSORS tensors.
hipError_t launch_quant_w(const WTensor *t, int64_t count, int mode, hipStream_t stream)
{
    WTensor part[QW_MAX_TENSORS];
    for (int bw = 4; bw >= 1; bw /= 2) {
        int64_t n = 0;
        for (int64_t j = 0; j <= count; ++j) {
            const bool take = j < count && (t[j].K / 128) % bw == 0 && (bw == 4 || (t[j].K / 128) % (2 * bw) != 0);
            if (take)
                part[n++] = t[j];
            if (n == QW_MAX_TENSORS || (j == count && n > 0)) {
                const hipError_t e = bw == 4   ? launch_quant_w_bw<4>(part, n, mode, stream)
                                     : bw == 2 ? launch_quant_w_bw<2>(part, n, mode, stream)
                                               : launch_quant_w_bw<1>(part, n, mode, stream);
                if (e != hipSuccess)
                    return e;
                n = 0;
            }
        }
    }
    return hipSuccess;
}

// ---- weights for training: codes of W and of its transpose in one pass ----------
//
// The backward pass multiplies by W^T (dX = dY W), whose 128x128 blocks are
// those of W transposed: block (kb, nb) of W^T holds the same 16384 values as
// block (nb, kb) of W, so its amax, scale and codes are the same, moved.  One
// read of the bf16 block therefore yields both operand sets, 4 bytes of
// traffic per element against 6 for two separate passes.  The workgroup
// loads the block as quant_w_kernel<MODE, 1> does, except that thread t
// covers 16-byte chunk (t % 16) of the 8 consecutive rows 8 (t / 16) .. + 7 -- an 8x8 byte
// square of codes, which it transposes in registers (byte permutes) into 8
// row pieces of the transposed block, each 8 contiguous bytes, gathered into
// whole rows through LDS.
struct QWDArgs {
    int count;
    int64_t tile_begin[QW_MAX_TENSORS + 1];
    const uint16_t *w[QW_MAX_TENSORS];
    uint8_t *q[QW_MAX_TENSORS];
    float *s[QW_MAX_TENSORS];
    uint8_t *qt[QW_MAX_TENSORS];
    float *st[QW_MAX_TENSORS];
    int64_t N[QW_MAX_TENSORS];
    int64_t K[QW_MAX_TENSORS];
};

// Transpose of an 8x8 byte square: row j is (lo[j], hi[j]) (bytes 0-3, 4-7);
// on return row i of the result holds byte i of every input row.
__device__ __forceinline__ void transpose8x8(const uint32_t (&lo)[8], const uint32_t (&hi)[8], uint32_t (&olo)[8],
                                             uint32_t (&ohi)[8])
{
    // 4x4 byte squares: (rows 0-3 | 4-7) x (bytes 0-3 | 4-7).  Within a square
    // first interleave the bytes of row pairs, then the halves of the pairs.
    // __builtin_amdgcn_perm(a, b, sel): byte k of the result is byte sel_k of
    // the 8-byte value a:b (0-3 from b, 4-7 from a).
    auto square = [](uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3, uint32_t &c0, uint32_t &c1, uint32_t &c2,
                     uint32_t &c3) {
        const uint32_t a_lo = __builtin_amdgcn_perm(r1, r0, 0x05010400u); // r0.b0 r1.b0 r0.b1 r1.b1
        const uint32_t a_hi = __builtin_amdgcn_perm(r1, r0, 0x07030602u); // r0.b2 r1.b2 r0.b3 r1.b3
        const uint32_t b_lo = __builtin_amdgcn_perm(r3, r2, 0x05010400u);
        const uint32_t b_hi = __builtin_amdgcn_perm(r3, r2, 0x07030602u);
        c0 = __builtin_amdgcn_perm(b_lo, a_lo, 0x05040100u); // r0.b0 r1.b0 r2.b0 r3.b0
        c1 = __builtin_amdgcn_perm(b_lo, a_lo, 0x07060302u);
        c2 = __builtin_amdgcn_perm(b_hi, a_hi, 0x05040100u);
        c3 = __builtin_amdgcn_perm(b_hi, a_hi, 0x07060302u);
    };
    // output row i < 4 takes byte i of lo[j]; i >= 4 byte i - 4 of hi[j];
    // its bytes 0-3 come from input rows 0-3, bytes 4-7 from rows 4-7
    square(lo[0], lo[1], lo[2], lo[3], olo[0], olo[1], olo[2], olo[3]);
    square(lo[4], lo[5], lo[6], lo[7], ohi[0], ohi[1], ohi[2], ohi[3]);
    square(hi[0], hi[1], hi[2], hi[3], olo[4], olo[5], olo[6], olo[7]);
    square(hi[4], hi[5], hi[6], hi[7], ohi[4], ohi[5], ohi[6], ohi[7]);
}

template <int MODE>
__global__ __launch_bounds__(QW_THREADS) void quant_w_dual_kernel(QWDArgs a)
{
    __shared__ uint32_t red[QW_THREADS / 64];
    __shared__ __attribute__((aligned(16))) uint8_t tl[128 * 128]; // the transposed code block
    const int64_t tile = blockIdx.x;
    int i = 0;
    while (i + 1 < a.count && tile >= a.tile_begin[i + 1])
        ++i;
    const int64_t N = a.N[i], K = a.K[i];
    const int64_t KB = K / 128, NB = N / 128;
    const int64_t local = tile - a.tile_begin[i];
    const int64_t nb = local / KB, kb = local % KB;

    const int t = threadIdx.x;
    const int rg = t >> 4, c = t & 15; // rows 8 rg .. 8 rg + 7, columns 8 c .. 8 c + 7 of the block
    const int64_t base = (nb * 128 + 8 * rg) * K + kb * 128 + c * 8;
    const uint16_t *w = a.w[i];

    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = __builtin_nontemporal_load((const u32x4 *)(w + base + j * K));

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
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const u32x2 codes = quant_chunk<MODE>(v[j], bq);
        __builtin_nontemporal_store(codes, (u32x2 *)(q + base + j * K));
        lo[j] = codes.x;
        hi[j] = codes.y;
    }
    // transposed block (kb, nb) of W^T [K, N]: its row 8 c + r holds column
    // 8 c + r of this block, whose bytes 8 rg .. 8 rg + 7 this thread holds.
    // The 16 KiB block is assembled in LDS so that each store instruction
    // writes whole 128-byte rows (stored straight from the 8x8 squares, a
    // wave instruction wrote 16 scattered 32-byte pieces and the kernel ran
    // at a third of the bandwidth).  LDS row p holds transposed row p, its
    // 8-byte piece g at slot g ^ (p / 8): the 16 lanes of a write that share
    // a piece index then fall in different banks.
    uint32_t tlo[8], thi[8];
    transpose8x8(lo, hi, tlo, thi);
#pragma unroll
    for (int r = 0; r < 8; ++r)
        *(u32x2 *)(tl + (8 * c + r) * 128 + ((rg ^ c) << 3)) = u32x2{tlo[r], thi[r]};
    __syncthreads();
    uint8_t *qt = a.qt[i];
    const int64_t tbase = kb * 128 * N + nb * 128;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        // 16-byte piece cc of transposed row tr, i.e. logical pieces 2 cc and
        // 2 cc + 1, stored at slots (2 cc) ^ g and (2 cc + 1) ^ g (g = tr / 8):
        // one aligned pair, in reverse order when g is odd
        const int idx = p * QW_THREADS + t;
        const int tr = idx >> 3, cc = idx & 7, g = tr >> 3;
        u32x4 d = *(const u32x4 *)(tl + tr * 128 + ((((2 * cc) ^ g) >> 1) << 4));
        if (g & 1)
            d = u32x4{d.z, d.w, d.x, d.y};
        __builtin_nontemporal_store(d, (u32x4 *)(qt + tbase + tr * N + cc * 16));
    }
    if (t == 0) {
        a.s[i][nb * KB + kb] = bq.s;
        a.st[i][kb * NB + nb] = bq.s;
    }
}

hipError_t launch_quant_w_dual(const WTensor *t, int64_t count, int mode, hipStream_t stream)
{
    for (int64_t first = 0; first < count; first += QW_MAX_TENSORS) {
        QWDArgs a = {};
        const int64_t n = (count - first) < QW_MAX_TENSORS ? (count - first) : QW_MAX_TENSORS;
        int64_t tiles = 0;
        for (int64_t j = 0; j < n; ++j) {
            const WTensor &wt = t[first + j];
            a.tile_begin[j] = tiles;
            a.w[j] = (const uint16_t *)wt.w;
            a.q[j] = (uint8_t *)wt.q;
            a.s[j] = wt.s;
            a.qt[j] = (uint8_t *)wt.qt;
            a.st[j] = wt.st;
            a.N[j] = wt.N;
            a.K[j] = wt.K;
            tiles += (wt.N / 128) * (wt.K / 128);
        }
        a.tile_begin[n] = tiles;
        a.count = (int)n;
        if (tiles == 0)
            continue;
        hipError_t e = (mode == SCALE_POW2) ? launch(quant_w_dual_kernel<SCALE_POW2>, dim3((unsigned)tiles),
                                                     dim3(QW_THREADS), 0, stream, a)
                                            : launch(quant_w_dual_kernel<SCALE_EXACT>, dim3((unsigned)tiles),
                                                     dim3(QW_THREADS), 0, stream, a);
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

// ---- activations for the weight gradient: 1x128 blocks along the rows ---------
//
// The weight gradient dW = dY^T X contracts over the tokens (the rows of X
// and of dY), so both operands are quantized in 1x128 blocks that run down a
// column: the quantization of X^T by quant_act_1x128's rule, written as X^T
// [K, M] with the tokens contiguous.  A workgroup takes a 128 x 128 tile of X
// (rows mb, columns kb): thread t loads chunk (t % 16) of rows
// 8 (t / 16) .. + 7, transposes that 8x8 square of bf16 values in registers
// and writes its 8 transposed row pieces into an LDS tile (piece g of row p
// at slot g ^ (p / 8), so the 16 lanes of a write and of a read that share a
// row or a piece index hit different banks).  The tile's 128 rows of X^T are
// then 1x128 blocks, quantized exactly as quant_act_kernel does: a 16-lane
// DPP row per block, one 16-byte chunk per lane.
// ROWS: also the ordinary 1x128 quantization of X (codes [M, K], scales
// [M, K/128]) from the same read.  Each row of the tile is one block whose
// 128 values sit in the 16 consecutive lanes that share 8 rows, so it is the
// activation quantizer's 16-lane block once more, before the transpose.
template <int MODE, bool ROWS = false>
__global__ __launch_bounds__(QW_THREADS) void quant_act_t_kernel(const uint16_t *__restrict__ x, uint8_t *__restrict__ q,
                                                                 float *__restrict__ s, int64_t M, int64_t K,
                                                                 uint8_t *__restrict__ qr = nullptr,
                                                                 float *__restrict__ sr = nullptr)
{
    __shared__ __attribute__((aligned(16))) uint8_t tl[128 * 256]; // the transposed bf16 tile
    const int64_t KB = K / 128, MB = M / 128;
    // Tiles walk M fastest, over XCD-contiguous ranges: a tile writes 128-byte
    // pieces of 128 rows of X^T's codes and one scale per row, and the tiles of
    // one XCD then continue each other's rows through its L2 (against K-first
    // tiles dealt round-robin: 11-24% faster from K = 14336 up, the same below)
    int64_t mb, kb;
    {
        const int64_t n = MB * KB, x = blockIdx.x % 8, i = blockIdx.x / 8, qn = n / 8, r = n % 8;
        const int64_t tile = x * qn + (x < r ? x : r) + i; // XCD x: [x qn + min(x, r), ...)
        mb = tile % MB;
        kb = tile / MB;
    }
    const int t = threadIdx.x;
    const int rg = t >> 4, c = t & 15;
    const int64_t base = (mb * 128 + 8 * rg) * K + kb * 128 + c * 8;

    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = __builtin_nontemporal_load((const u32x4 *)(x + base + j * K));
    if constexpr (ROWS) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            BlockQuant<MODE> bq;
            bq.init(amax_value(row16_max(chunk_max_mag(v[j]))));
            *(u32x2 *)(qr + base + j * K) = quant_chunk<MODE>(v[j], bq); // (cached: a GEMM operand next)
            if (c == 0)
                sr[(mb * 128 + 8 * rg + j) * KB + kb] = bq.s;
        }
    }
    // transposed row i (column 8 c + i of the tile) holds element i of rows
    // 8 rg .. 8 rg + 7; its dword p pairs rows 2p (low half) and 2p + 1
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
        u32x4 o;
        o.x = __builtin_amdgcn_perm(v[1][i >> 1], v[0][i >> 1], sel);
        o.y = __builtin_amdgcn_perm(v[3][i >> 1], v[2][i >> 1], sel);
        o.z = __builtin_amdgcn_perm(v[5][i >> 1], v[4][i >> 1], sel);
        o.w = __builtin_amdgcn_perm(v[7][i >> 1], v[6][i >> 1], sel);
        const int p = 8 * c + i;
        *(u32x4 *)(tl + p * 256 + ((rg ^ c) << 4)) = o;
    }
    __syncthreads();

    const int lane = t & 63, wave = t >> 6;
    const int g = lane & 15; // 16-byte chunk (8 tokens) of the block
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
        const int p = pass * 16 + wave * 4 + (lane >> 4); // row of X^T within the tile
        const u32x4 val = *(const u32x4 *)(tl + p * 256 + ((g ^ (p >> 3)) << 4));
        const float amax = amax_value(row16_max(chunk_max_mag(val)));
        BlockQuant<MODE> bq;
        bq.init(amax);
        const u32x2 codes = quant_chunk<MODE>(val, bq);
        const int64_t row = kb * 128 + p;
        *(u32x2 *)(q + row * M + mb * 128 + 8 * g) = codes; // (cached: the weight gradient's operand next)
        if (g == 0)
            s[row * MB + mb] = bq.s;
    }
}

hipError_t launch_quant_act_t(const void *x, int64_t M, int64_t K, void *xqt, float *xst, int mode,
                              hipStream_t stream, void *xq, float *xs)
{
    const int64_t tiles = (M / 128) * (K / 128);
    if (tiles == 0)
        return hipSuccess;
    const dim3 g((unsigned)tiles), b(QW_THREADS);
    const uint16_t *xp = (const uint16_t *)x;
    uint8_t *qt = (uint8_t *)xqt, *qr = (uint8_t *)xq;
    if (xq != nullptr) {
        if (mode == SCALE_POW2)
            return launch(quant_act_t_kernel<SCALE_POW2, true>, g, b, 0, stream, xp, qt, xst, M, K, qr, xs);
        return launch(quant_act_t_kernel<SCALE_EXACT, true>, g, b, 0, stream, xp, qt, xst, M, K, qr, xs);
    }
    if (mode == SCALE_POW2)
        return launch(quant_act_t_kernel<SCALE_POW2, false>, g, b, 0, stream, xp, qt, xst, M, K, qr, xs);
    return launch(quant_act_t_kernel<SCALE_EXACT, false>, g, b, 0, stream, xp, qt, xst, M, K, qr, xs);
}

} // namespace fp8bs
