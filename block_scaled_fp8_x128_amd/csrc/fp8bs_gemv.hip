// fp8bs_gemv.hip -- the block-scaled product for one activation row (rollout
// decode at one token), on the vector ALUs.
//
// The article "NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
// precision training", section "Technical breakthrough": linear layers run FP8
// math on operands quantized per 1x128 (activations) and 128x128 (weights)
// block; section "Real-world performance gains": generation (rollout) runs in
// FP8 too.  With a single activation row,
//   Y[0, n] = sum_kb ws[n/128, kb] * sum_{k in kb} (decode(xq[k]) * xs[kb]) * decode(wq[n, k]),
// is bound by streaming W from HBM, and a matrix-core tile would be 1/16
// useful while its operand layout forces half-line loads (16 rows x 64 bytes
// per wave instruction).  Here every wave instruction reads 1 KiB of one W
// row, contiguous:
//   - wave w of a workgroup owns K chunk w (bytes 1024 w .. 1024 w + 1023 of
//     every row); lane l holds the 16 activation values k = 1024 w + 16 l ..
//     + 15, decoded and multiplied by their block's scale once;
//   - per W row, the lane decodes its 16 codes (v_cvt_pk_f32_fp8), sums the
//     16 products by fp32 FMAs in k order and multiplies the sum by the
//     row block's weight scale for its K block (8 lanes share a block);
//   - 8 rows at a time, the 64 lane partials of each row are summed by a
//     transposing butterfly (10 lane exchanges for 8 rows), and the per-wave
//     row sums are added over the waves in wave order through LDS.
// Every reduction has a fixed order, so results are deterministic.  The
// products and sums are plain fp32, with no matrix-core accumulation: the
// result differs from the matrix-core path by rounding only, and of the two
// it is the closer to the exact value (the matrix cores sum a K block's
// products at reduced precision when one of them dominates).
//
// QX = 1 / 2: the activation row arrives as bf16 and each 8-lane group
// quantizes its 128-value block with the 1x128 quantizer's own encoder
// (EXACT / POW2): the same codes and scale quant_act_1x128 writes, hence the
// same activation values and Y bit for bit as that quantizer followed by the
// QX = 0 kernel.
#include "fp8bs_device.hpp"
#include "fp8bs_internal.hpp"

namespace fp8bs {

constexpr int GV_MAX_WAVES = 16; // one 1 KiB chunk of K per wave: K <= 16384

struct GemvArgs {
    const void *x;    // QX = 0: E4M3 codes [K]; QX > 0: bf16 [K]
    const float *xs;  // QX = 0: activation scales [K/128]
    const uint8_t *wq;
    const float *ws;
    void *y;
    int64_t N, K;
};

typedef float f2 __attribute__((ext_vector_type(2)));

// 16 E4M3 codes (one 16-byte load) -> 16 floats, exactly.
__device__ __forceinline__ void decode16(const u32x4 &c, float (&v)[16])
{
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], false);
        const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[d], true);
        v[4 * d + 0] = lo.x;
        v[4 * d + 1] = lo.y;
        v[4 * d + 2] = hi.x;
        v[4 * d + 3] = hi.y;
    }
}

template <int ROWS, bool OUT_F32, int QX>
__global__ __launch_bounds__(GV_MAX_WAVES * 64) void gemv_kernel(GemvArgs a)
{
    static_assert(ROWS % 8 == 0 && 128 % ROWS == 0, "row groups of 8 inside one 128-row weight block");
    __shared__ float red[GV_MAX_WAVES][ROWS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int64_t K = a.K, KB = K / 128;
    const int64_t row0 = (int64_t)blockIdx.x * ROWS;
    const int64_t k0 = (int64_t)wave * 1024 + lane * 16;
    const bool live = k0 < K; // (K % 128 == 0: a 128-value block is live or dead as a whole)
    const int64_t kl = live ? k0 : 0;

    // ---- this lane's 16 activation values, decoded and scaled ----
    float xv[16];
    if constexpr (QX == 0) {
        const u32x4 c = live ? *(const u32x4 *)((const uint8_t *)a.x + kl) : u32x4{0u, 0u, 0u, 0u};
        decode16(c, xv);
        const float s = live ? a.xs[kl / 128] : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            xv[i] *= s;
    } else {
        constexpr int MODE = QX == 2 ? SCALE_POW2 : SCALE_EXACT;
        const u32x4 *xp = (const u32x4 *)((const uint16_t *)a.x + kl);
        const u32x4 b0 = live ? xp[0] : u32x4{0u, 0u, 0u, 0u};
        const u32x4 b1 = live ? xp[1] : u32x4{0u, 0u, 0u, 0u};
        // the block's 128 values sit in 8 consecutive lanes
        uint32_t m = chunk_max_mag(b0);
        const uint32_t m1 = chunk_max_mag(b1);
        m = m > m1 ? m : m1;
#pragma unroll
        for (int sh = 1; sh < 8; sh <<= 1) {
            const uint32_t o = (uint32_t)__shfl_xor((int)m, sh);
            m = m > o ? m : o;
        }
        BlockQuant<MODE> bq;
        bq.init(amax_value(m));
        const u32x2 q0 = quant_chunk<MODE>(b0, bq);
        const u32x2 q1 = quant_chunk<MODE>(b1, bq);
        decode16(u32x4{q0.x, q0.y, q1.x, q1.y}, xv);
        const float s = live ? bq.s : 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            xv[i] *= s;
    }
    // the weight scale of rows row0 .. row0 + ROWS - 1 (one 128-row block) for this lane's K block
    const float wsl = live ? a.ws[(row0 / 128) * KB + kl / 128] : 0.0f;

    // ---- W rows, 8 at a time, loads of the next 8 in flight ----
    const uint8_t *wrow = a.wq + row0 * K + kl;
    constexpr int G = ROWS / 8;
    u32x4 buf[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        buf[0][j] = __builtin_nontemporal_load((const u32x4 *)(wrow + (int64_t)j * K));
#pragma unroll
    for (int g = 0; g < G; ++g) {
        if (g + 1 < G) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                buf[(g + 1) & 1][j] = __builtin_nontemporal_load((const u32x4 *)(wrow + (int64_t)(8 * (g + 1) + j) * K));
        }
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float wv[16];
            decode16(buf[g & 1][j], wv);
            float acc = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i)
                acc = __builtin_fmaf(xv[i], wv[i], acc);
            p[j] = acc * wsl;
        }
        // transposing butterfly: lanes with bit 5 (4, 3) of their id set keep
        // the upper half of the remaining rows and send the lower half, so
        // after three halvings lane l holds row l / 8 summed over its 8-lane
        // group's partners; three more exchanges finish the 64-lane sums
        {
            const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
            float q[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float send = b5 ? p[j] : p[j + 4];
                const float keep = b5 ? p[j + 4] : p[j];
                q[j] = keep + __shfl_xor(send, 32);
            }
            float r[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float send = b4 ? q[j] : q[j + 2];
                const float keep = b4 ? q[j + 2] : q[j];
                r[j] = keep + __shfl_xor(send, 16);
            }
            const float send = b3 ? r[0] : r[1];
            const float keep = b3 ? r[1] : r[0];
            float t = keep + __shfl_xor(send, 8);
            t += __shfl_xor(t, 4);
            t += __shfl_xor(t, 2);
            t += __shfl_xor(t, 1);
            if ((lane & 7) == 0)
                red[wave][8 * g + (lane >> 3)] = t;
        }
    }
    __syncthreads();
    if (threadIdx.x < ROWS) {
        const int r = threadIdx.x;
        float s = 0.0f;
        for (int w = 0; w < nw; ++w)
            s += red[w][r];
        if constexpr (OUT_F32)
            ((float *)a.y)[row0 + r] = s;
        else
            ((__bf16 *)a.y)[row0 + r] = (__bf16)s;
    }
}

bool gemv_ok(int64_t M, int64_t N, int64_t K)
{
    return M == 1 && N % 128 == 0 && K % 128 == 0 && K <= (int64_t)GV_MAX_WAVES * 1024 && N * K < ((int64_t)1 << 40);
}

template <int ROWS, int QX>
static hipError_t run_gemv(const GemvArgs &a, bool out_f32, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.N / ROWS)), block((unsigned)(((a.K + 1023) / 1024) * 64));
    if (out_f32)
        return launch(gemv_kernel<ROWS, true, QX>, grid, block, 0, stream, a);
    return launch(gemv_kernel<ROWS, false, QX>, grid, block, 0, stream, a);
}

// Rows per workgroup: 32 while that still leaves two workgroups per compute
// unit, else 16, else 8.
template <int QX>
static hipError_t run_gemv_rows(const GemvArgs &a, bool out_f32, hipStream_t stream)
{
    if (a.N / 32 >= 512)
        return run_gemv<32, QX>(a, out_f32, stream);
    if (a.N / 16 >= 256)
        return run_gemv<16, QX>(a, out_f32, stream);
    return run_gemv<8, QX>(a, out_f32, stream);
}

hipError_t launch_gemv(const void *x, const float *xs, const void *wq, const float *ws, int64_t N, int64_t K, void *y,
                       int out_fp32, int quantize, hipStream_t stream)
{
    GemvArgs a = {x, xs, (const uint8_t *)wq, ws, y, N, K};
    if (quantize == 1)
        return run_gemv_rows<1>(a, out_fp32 != 0, stream);
    if (quantize == 2)
        return run_gemv_rows<2>(a, out_fp32 != 0, stream);
    return run_gemv_rows<0>(a, out_fp32 != 0, stream);
}

} // namespace fp8bs
