// fp8bs_attn.hip -- attention of one new query token over an FP8 KV cache
// (rollout decode), gfx950.
//
// The article "NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
// precision training", section "Real-world performance gains": keeping the KV
// cache and attention in FP8 as well lifts the end-to-end gain from 15-25% to
// about 48%.  The cache here holds keys and values as E4M3 codes with one fp32
// scale per (token, head): the 1x128 blocks of quant_act_1x128 over the
// [tokens, heads * 128] rows.  For query head h of sequence b (key/value head
// g = h / (Hq / Hkv)):
//   s_j = sm_scale * ks[b, j, g] * sum_d q[b, h, d] * decode(kq[b, j, g, d]),  j < len_b,
//   o[b, h, :] = sum_j softmax(s)_j * vs[b, j, g] * decode(vq[b, j, g, :]).
//
// Decode attention reads every cached byte once per step and does little
// arithmetic per byte, so the cache bandwidth bounds it; FP8 halves those
// bytes against bf16.  Work split: workgroup (b * Hkv + g, split) takes the
// tokens [split * chunk, min((split + 1) * chunk, len_b)) of one key/value
// head for all G = Hq / Hkv of its query heads; its 4 waves take 16-token
// tiles in turn, each keeping its own running softmax (max, sum, output).
//   scores: the tile's key codes become bf16 (exact: every E4M3 value is a
//     bf16) and one v_mfma_f32_16x16x32_bf16 per 32 dimensions multiplies them
//     by the query heads (bf16 products are exact in fp32); the key scale and
//     sm_scale * log2(e) follow in fp32, and exp2 replaces exp;
//   values: each lane owns 8 dimensions of every fourth token of the tile and
//     accumulates p * vs * decode(v) for the G heads in fp32, p coming from the
//     scores through the wave's LDS area.
// The waves' states merge through LDS; with several splits per sequence a
// second kernel merges the splits' (max, sum, output) in split order.  Every
// order is fixed, so results are deterministic.
#include "fp8bs_device.hpp"
#include "fp8bs_internal.hpp"

namespace fp8bs {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));

constexpr int AD = 128;       // head dimension (one 1x128 scale block)
constexpr int ATT_WAVES = 4;
constexpr float kLog2e = 1.4426950408889634f;

struct AttnArgs {
    const uint16_t *q;   // [B, Hq, 128] bf16
    const uint8_t *kq;   // [B, T, Hkv, 128]
    const float *ks;     // [B, T, Hkv]
    const uint8_t *vq;
    const float *vs;
    const int32_t *lens; // [B]
    void *out;           // [B, Hq, 128]
    float *part;         // splits > 1: [B * Hq, splits, 2 + 128] (max, sum, output)
    int64_t B, T, Hq, Hkv;
    int chunk;           // tokens per split (a multiple of 64)
    int splits;
    float scale_log2;    // sm_scale * log2(e)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t attn_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes >= 0x7fffffffLL ? 0x7fffffff : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, 0x00020000);
}

// 8 E4M3 codes (two dwords) -> 8 bf16, in byte order.
__device__ __forceinline__ bf8v codes_to_bf16(uint32_t w0, uint32_t w1)
{
    const bf2v a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
    const bf2v b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
    const bf2v c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
    const bf2v d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
    return bf8v{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

// LDS of one workgroup: per wave the tile's p * vs [16 tokens][G] and the
// heads' rescale factors; then the waves' final states for the merge.
template <int G>
struct AttnLds {
    float pv[ATT_WAVES][16 * G];
    float alpha[ATT_WAVES][G];
    float m[ATT_WAVES][G];
    float l[ATT_WAVES][G];
    float o[ATT_WAVES][G][AD];
};

template <int G, bool OUT_F32, bool SPLIT>
__global__ __launch_bounds__(ATT_WAVES * 64) void kv_attn_decode_kernel(AttnArgs a)
{
    __shared__ AttnLds<G> sh;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t bg = blockIdx.x;
    const int64_t b = bg / a.Hkv, g = bg % a.Hkv;
    const int split = blockIdx.y;
    int64_t len = a.lens[b];
    len = len < 0 ? 0 : (len > a.T ? a.T : len);
    const int64_t t0 = (int64_t)split * a.chunk;
    const int64_t t1 = (t0 + a.chunk) < len ? (t0 + a.chunk) : len;
    const int64_t rowb = a.Hkv * AD; // bytes between consecutive tokens of one head

    // query fragments (MFMA B operand): lane (n = lane % 16, grp = lane / 16)
    // holds the 8 dimensions 32 grp + 8 s .. + 7 of query head g G + n for
    // MFMA s (heads n >= G are zero); the key fragments below use the same
    // dimension order, so each MFMA s sums over its 32 dimensions once
    const int n = lane & 15, grp = lane >> 4;
    bf8v qf[4];
    {
        const uint16_t *qh = a.q + ((b * a.Hq) + g * G + (n < G ? n : 0)) * AD + 32 * grp;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 w = (n < G) ? *(const u32x4 *)(qh + 8 * s) : u32x4{0u, 0u, 0u, 0u};
            qf[s] = __builtin_bit_cast(bf8v, w);
        }
    }
    const __amdgpu_buffer_rsrc_t kr = attn_rsrc(a.kq + ((b * a.T) * a.Hkv + g) * AD, len * rowb);
    const __amdgpu_buffer_rsrc_t vr = attn_rsrc(a.vq + ((b * a.T) * a.Hkv + g) * AD, len * rowb);
    const float *ksb = a.ks + (b * a.T) * a.Hkv + g;
    const float *vsb = a.vs + (b * a.T) * a.Hkv + g;

    // the softmax state of head (lane % 16) (meaningful for heads < G) ...
    float mh = -INFINITY, lh = 0.0f;
    // ... and the output partials: lane (ts = lane / 16, c = lane % 16) sums
    // tokens ts, ts + 4, ts + 8, ts + 12 of each tile into dims 8 c .. 8 c + 7
    const int ts = grp, d0 = 8 * n;
    float o[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[h][e] = 0.0f;

    for (int64_t tb = t0 + 16 * wave; tb < t1; tb += 16 * ATT_WAVES) {
        // ---- scores of tokens tb .. tb + 15 against the G heads ----
        // A operand: lane (t = lane % 16, grp) holds bytes 32 grp .. + 31 of token tb + t
        const int koff = (int)((tb + n) * rowb) + 32 * grp;
        const u32x4 k0 = __builtin_amdgcn_raw_buffer_load_b128(kr, koff, 0, 0);
        const u32x4 k1 = __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 16, 0, 0);
        // the tile's key and value scales: lane t < 16 loads token tb + t's
        const bool tok_ok = n + tb < t1;
        const float ksv = (lane < 16 && tok_ok) ? ksb[(tb + n) * a.Hkv] : 0.0f;
        const float vsv = (lane < 16 && tok_ok) ? vsb[(tb + n) * a.Hkv] : 0.0f;
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(k0.x, k0.y), qf[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(k0.z, k0.w), qf[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(k1.x, k1.y), qf[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16(k1.z, k1.w), qf[3], acc, 0, 0, 0);
        // lane (grp, n) holds tokens tb + 4 grp + r of head n; scores in log2 units
        float s[4], p[4];
        float mt = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * grp + r;
            const float kscale = __shfl(ksv, t);
            s[r] = (tb + t < t1) ? acc[r] * kscale * a.scale_log2 : -INFINITY;
            mt = mt > s[r] ? mt : s[r];
        }
        float x = __shfl_xor(mt, 16);
        mt = mt > x ? mt : x;
        x = __shfl_xor(mt, 32);
        mt = mt > x ? mt : x;
        const float mnew = mh > mt ? mh : mt; // finite: the tile holds a token below t1
        const float alpha = __builtin_amdgcn_exp2f(mh - mnew);
        float ps = 0.0f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            p[r] = __builtin_amdgcn_exp2f(s[r] - mnew);
            ps += p[r];
        }
        ps += __shfl_xor(ps, 16);
        ps += __shfl_xor(ps, 32);
        lh = lh * alpha + ps;
        mh = mnew;
        // p * vs of each (token, head) and the heads' rescale factors to the
        // wave's LDS (the shuffles run on every lane, outside the branch)
        float vsr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            vsr[r] = __shfl(vsv, 4 * grp + r);
        if (n < G) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sh.pv[wave][(4 * grp + r) * G + n] = p[r] * vsr[r];
            if (grp == 0)
                sh.alpha[wave][n] = alpha;
        }
        // ---- values: tokens ts + 4 u of the tile, dims d0 .. d0 + 7 ----
        uint32_t vw[4][2];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = ts + 4 * u;
            const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(vr, (int)((tb + t) * rowb) + d0, 0, 0);
            const bool ok = tb + t < t1;
            vw[u][0] = ok ? w.x : 0u;
            vw[u][1] = ok ? w.y : 0u;
        }
        // (LDS writes and reads of one wave complete in order)
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const float al = sh.alpha[wave][h];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[h][e] *= al;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int t = ts + 4 * u;
            float v[8];
            const f2v v01 = __builtin_amdgcn_cvt_pk_f32_fp8(vw[u][0], false);
            const f2v v23 = __builtin_amdgcn_cvt_pk_f32_fp8(vw[u][0], true);
            const f2v v45 = __builtin_amdgcn_cvt_pk_f32_fp8(vw[u][1], false);
            const f2v v67 = __builtin_amdgcn_cvt_pk_f32_fp8(vw[u][1], true);
            v[0] = v01.x, v[1] = v01.y, v[2] = v23.x, v[3] = v23.y;
            v[4] = v45.x, v[5] = v45.y, v[6] = v67.x, v[7] = v67.y;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pw = sh.pv[wave][t * G + h];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[h][e] = __builtin_fmaf(pw, v[e], o[h][e]);
            }
        }
    }

    // ---- the wave's state: sum the four token groups' partials ----
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            o[h][e] += __shfl_xor(o[h][e], 16);
            o[h][e] += __shfl_xor(o[h][e], 32);
        }
    if (lane < G) {
        sh.m[wave][lane] = mh;
        sh.l[wave][lane] = lh;
    }
    if (grp == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sh.o[wave][h][d0 + e] = o[h][e];
    }
    __syncthreads();

    // ---- merge the waves (in wave order): thread i handles dims of head i / 64 ... ----
    for (int idx = threadIdx.x; idx < G * (AD / 2); idx += ATT_WAVES * 64) {
        const int h = idx / (AD / 2), d = 2 * (idx % (AD / 2));
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < ATT_WAVES; ++w)
            M = M > sh.m[w][h] ? M : sh.m[w][h];
        float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < ATT_WAVES; ++w) {
                const float f = __builtin_amdgcn_exp2f(sh.m[w][h] - M); // 0 for an empty wave
                L = __builtin_fmaf(f, sh.l[w][h], L);
                o0 = __builtin_fmaf(f, sh.o[w][h][d], o0);
                o1 = __builtin_fmaf(f, sh.o[w][h][d + 1], o1);
            }
        }
        const int64_t bh = b * a.Hq + g * G + h;
        if constexpr (SPLIT) {
            float *pp = a.part + (bh * a.splits + split) * (2 + AD);
            if (d == 0) {
                pp[0] = M;
                pp[1] = L;
            }
            pp[2 + d] = o0;
            pp[2 + d + 1] = o1;
        } else {
            const float r0 = L > 0.0f ? o0 / L : 0.0f, r1 = L > 0.0f ? o1 / L : 0.0f;
            if constexpr (OUT_F32) {
                *(f2v *)((float *)a.out + bh * AD + d) = f2v{r0, r1};
            } else {
                const bf2v v = __builtin_convertvector(f2v{r0, r1}, bf2v);
                *(bf2v *)((__bf16 *)a.out + bh * AD + d) = v;
            }
        }
    }
}

// Merge of the splits of one (sequence, query head): one wave each, lane l
// takes dims 2 l and 2 l + 1; the splits are added in split order.
template <bool OUT_F32>
__global__ __launch_bounds__(64) void kv_attn_combine_kernel(const float *part, int splits, void *out)
{
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    const float *pp = part + bh * splits * (2 + AD);
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s)
        M = M > pp[s * (2 + AD)] ? M : pp[s * (2 + AD)];
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    if (M != -INFINITY) {
        for (int s = 0; s < splits; ++s) {
            const float *q = pp + s * (2 + AD);
            const float f = __builtin_amdgcn_exp2f(q[0] - M);
            L = __builtin_fmaf(f, q[1], L);
            o0 = __builtin_fmaf(f, q[2 + 2 * lane], o0);
            o1 = __builtin_fmaf(f, q[3 + 2 * lane], o1);
        }
    }
    const float r0 = L > 0.0f ? o0 / L : 0.0f, r1 = L > 0.0f ? o1 / L : 0.0f;
    if constexpr (OUT_F32) {
        *(f2v *)((float *)out + bh * AD + 2 * lane) = f2v{r0, r1};
    } else {
        *(bf2v *)((__bf16 *)out + bh * AD + 2 * lane) = __builtin_convertvector(f2v{r0, r1}, bf2v);
    }
}

// Splits per sequence: enough workgroups to cover the CUs twice, each split at
// least 256 tokens; the chunk is a multiple of the 4 waves' 16-token tiles.
static void attn_plan(int64_t B, int64_t T, int64_t Hkv, int &splits, int &chunk)
{
    const int64_t heads = B * Hkv;
    int64_t s = (512 + heads - 1) / heads;
    const int64_t smax = (T + 255) / 256;
    s = s < smax ? s : smax;
    s = s < 1 ? 1 : (s > 64 ? 64 : s);
    int64_t c = (T + s - 1) / s;
    c = (c + 63) / 64 * 64;
    s = (T + c - 1) / c;
    splits = (int)(s < 1 ? 1 : s);
    chunk = (int)(c < 64 ? 64 : c);
}

size_t kv_attention_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv)
{
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0)
        return 0;
    int splits, chunk;
    attn_plan(B, T, Hkv, splits, chunk);
    return splits > 1 ? (size_t)B * (size_t)Hq * (size_t)splits * (2 + AD) * sizeof(float) : 0;
}

template <int G>
static hipError_t run_attn(const AttnArgs &a, bool out_f32, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.B * a.Hkv), (unsigned)a.splits), block(ATT_WAVES * 64);
    if (a.splits > 1) {
        hipError_t e = launch(kv_attn_decode_kernel<G, false, true>, grid, block, 0, stream, a);
        if (e != hipSuccess)
            return e;
        if (out_f32)
            return launch(kv_attn_combine_kernel<true>, dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, stream,
                          (const float *)a.part, a.splits, a.out);
        return launch(kv_attn_combine_kernel<false>, dim3((unsigned)(a.B * a.Hq)), dim3(64), 0, stream,
                      (const float *)a.part, a.splits, a.out);
    }
    if (out_f32)
        return launch(kv_attn_decode_kernel<G, true, false>, grid, block, 0, stream, a);
    return launch(kv_attn_decode_kernel<G, false, false>, grid, block, 0, stream, a);
}

bool kv_attention_group_ok(int64_t Hq, int64_t Hkv)
{
    if (Hkv <= 0 || Hq % Hkv != 0)
        return false;
    const int64_t G = Hq / Hkv;
    return G == 1 || G == 2 || G == 4 || G == 8;
}

hipError_t launch_kv_attention(const void *q, const void *kq, const float *ks, const void *vq, const float *vs,
                               const int32_t *lens, int64_t B, int64_t T, int64_t Hq, int64_t Hkv, float sm_scale,
                               void *out, int out_fp32, void *workspace, hipStream_t stream)
{
    if (B == 0)
        return hipSuccess;
    AttnArgs a = {};
    a.q = (const uint16_t *)q;
    a.kq = (const uint8_t *)kq;
    a.ks = ks;
    a.vq = (const uint8_t *)vq;
    a.vs = vs;
    a.lens = lens;
    a.out = out;
    a.part = (float *)workspace;
    a.B = B;
    a.T = T;
    a.Hq = Hq;
    a.Hkv = Hkv;
    attn_plan(B, T, Hkv, a.splits, a.chunk);
    a.scale_log2 = sm_scale * kLog2e;
    switch (Hq / Hkv) {
    case 1:
        return run_attn<1>(a, out_fp32 != 0, stream);
    case 2:
        return run_attn<2>(a, out_fp32 != 0, stream);
    case 4:
        return run_attn<4>(a, out_fp32 != 0, stream);
    default:
        return run_attn<8>(a, out_fp32 != 0, stream);
    }
}

} // namespace fp8bs
