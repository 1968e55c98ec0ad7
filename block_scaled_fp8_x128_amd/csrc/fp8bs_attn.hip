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
// bytes against bf16.  Work split: workgroup (b * HG + hg, split) of S splits
// takes the 16-token tiles split, split + S, split + 2 S, ... below len_b of
// sequence b (so that the S workgroups of a sequence read neighbouring tiles
// at a time: 1.8-2.2% faster than contiguous token ranges per split) for
// the key/value heads 8 hg .. 8 hg + 7, one per wave, each wave serving all
// G = Hq / Hkv query heads of its key/value head and keeping their running
// softmax (max, sum, output).  The cache rows are [T, Hkv, 128]: stepping
// through 16-token tiles together, the waves of a workgroup read whole
// contiguous token rows, where one head alone would take 128 bytes of every
// Hkv * 128.
//   scores: the tile's key codes become bf16 (exact: every E4M3 value is a
//     bf16) and one v_mfma_f32_16x16x32_bf16 per 32 dimensions multiplies the
//     query heads by them (bf16 products are exact in fp32), heads down the
//     rows and tokens across the columns, so per-head max and sum over a tile
//     are DPP reductions within a 16-lane row; the key scale and
//     sm_scale * log2(e) follow in fp32, and exp2 replaces exp;
//   values: each lane owns 8 dimensions of every fourth token of the tile (4
//     dimensions of every second token for G = 8) and accumulates
//     p * vs * decode(v) for the G heads in fp32, p coming from the scores
//     through the wave's LDS area; the token groups' sums are added by lane
//     exchanges at the end.
// With several splits per sequence a second kernel merges the splits' (max,
// sum, output) in split order.  Every order is fixed, so results are
// deterministic.
#include "fp8bs_device.hpp"
#include "fp8bs_internal.hpp"

namespace fp8bs {

typedef __bf16 bf8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));

constexpr int AD = 128;       // head dimension (one 1x128 scale block)
constexpr int ATT_WAVES = 8;
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

// Max and sum over the 16 lanes of a DPP row; every lane of the row gets the
// result (the butterfly's partners: quad_perm [1,0,3,2], [2,3,0,1], then the
// row's half mirror and full mirror).
__device__ __forceinline__ float dpp_f(float v, int ctrl_id)
{
    const int x = __builtin_bit_cast(int, v);
    int t;
    switch (ctrl_id) {
    case 0: t = __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false); break;
    case 1: t = __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false); break;
    case 2: t = __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false); break;
    default: t = __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false); break;
    }
    return __builtin_bit_cast(float, t);
}
__device__ __forceinline__ float row16_fmax(float v)
{
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float t = dpp_f(v, c);
        v = v > t ? v : t;
    }
    return v;
}
__device__ __forceinline__ float row16_fsum(float v)
{
#pragma unroll
    for (int c = 0; c < 4; ++c)
        v += dpp_f(v, c);
    return v;
}

// LDS of one workgroup: per wave the tile's p * vs [16 tokens][G] and the
// heads' rescale factors.
template <int G>
struct AttnLds {
    float pv[ATT_WAVES][16 * G];
    float alpha[ATT_WAVES][G];
};

template <int G, bool OUT_F32, bool SPLIT>
__global__ __launch_bounds__(ATT_WAVES * 64) void kv_attn_decode_kernel(AttnArgs a)
{
    __shared__ AttnLds<G> sh;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t HG = (a.Hkv + ATT_WAVES - 1) / ATT_WAVES; // groups of 8 key/value heads
    const int64_t b = blockIdx.x / HG, g = (blockIdx.x % HG) * ATT_WAVES + wave;
    if (g >= a.Hkv)
        return; // (no barrier follows)
    const int split = blockIdx.y;
    int64_t len = a.lens[b];
    len = len < 0 ? 0 : (len > a.T ? a.T : len);
    const int64_t t0 = (int64_t)split * 16, tstride = (int64_t)a.splits * 16; // this split's tiles
    const int64_t t1 = len;
    const int64_t rowb = a.Hkv * AD; // bytes between consecutive tokens of one head

    // query fragments (MFMA A operand): lane (n = lane % 16, grp = lane / 16)
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
    // (the scales of tokens at or past len read as zeros, like the codes)
    const __amdgpu_buffer_rsrc_t ksr = attn_rsrc(a.ks + (b * a.T) * a.Hkv + g, len * a.Hkv * 4);
    const __amdgpu_buffer_rsrc_t vsr = attn_rsrc(a.vs + (b * a.T) * a.Hkv + g, len * a.Hkv * 4);

    // Scores come out of the MFMAs with heads down the rows and the tile's 16
    // tokens across the columns: lane (grp, n) holds heads 4 grp + r (r = 0
    // .. 3) of token tb + n.  A transpose of the 4 x 4 blocks of 16-lane rows
    // (three lane-row swaps) then gives lane (grp, n) heads 4 r + grp in its
    // registers r < R, so that the G heads fill the rows of R = ceil(G / 4)
    // registers instead of G of the 16 rows of four: a head's max and sum over
    // the tile stay reductions within one 16-lane row (DPP), each lane needs
    // only its own token's scales, and the softmax arithmetic runs on R
    // registers, not four.  The softmax state of head 4 r + grp is kept by
    // every lane of its row (meaningful for heads < G) ...
    constexpr int R = G > 4 ? 2 : 1;
    float mh[R], lh[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        mh[r] = -INFINITY;
        lh[r] = 0.0f;
    }
    // ... and the output partials: the lanes form TG token groups of LPG
    // lanes; lane (ts = lane / LPG, c = lane % LPG) sums tokens ts, ts + TG,
    // ... of each tile into dims DPL c .. DPL c + DPL - 1 of all G heads.
    // Four groups of 8 dims while G <= 4; two groups of 4 dims for G = 8,
    // which halves the G x DPL accumulators (64 -> 32 registers), so that two
    // workgroups of 8 waves still fit on a CU (at 4 x 8 the kernel needed
    // more than the 128 registers a wave may hold at four waves per SIMD)
    constexpr int TG = G > 4 ? 2 : 4, LPG = 64 / TG, DPL = 2 * TG, UPL = 16 / TG;
    const int ts = lane / LPG, d0 = DPL * (lane % LPG);
    float o[G][DPL];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e)
            o[h][e] = 0.0f;

    // The tile's operands, loaded one tile ahead: key bytes 32 grp .. + 31 of
    // token tb + n (B operand of the score MFMAs) with that token's key and
    // value scales, and value dims d0 .. d0 + DPL - 1 of tokens tb + ts + TG u.  Codes
    // and scales of tokens at or past the sequence's length read as zeros
    // (buffer range check).
    struct TileIn {
        u32x4 k0, k1;
        uint32_t v[UPL][DPL / 4];
        float ks, vs;
    };
    auto load_tile = [&](int64_t tb) {
        TileIn in;
        const int koff = (int)((tb + n) * rowb) + 32 * grp;
        in.k0 = __builtin_amdgcn_raw_buffer_load_b128(kr, koff, 0, 0);
        in.k1 = __builtin_amdgcn_raw_buffer_load_b128(kr, koff + 16, 0, 0);
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int off = (int)((tb + ts + TG * u) * rowb) + d0;
            if constexpr (DPL == 8) {
                const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(vr, off, 0, 0);
                in.v[u][0] = w.x;
                in.v[u][DPL / 4 - 1] = w.y;
            } else {
                in.v[u][0] = __builtin_amdgcn_raw_buffer_load_b32(vr, off, 0, 0);
            }
        }
        in.ks = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(ksr, (int)((tb + n) * a.Hkv * 4), 0, 0));
        in.vs = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(vsr, (int)((tb + n) * a.Hkv * 4), 0, 0));
        return in;
    };
    // (a tile at t1 or past it loads zeros and no scale)
    TileIn nxt = load_tile(t0 < t1 ? t0 : t1);
    for (int64_t tb = t0; tb < t1; tb += tstride) {
        const TileIn cur = nxt;
        // the next tile's loads go out before this tile's arithmetic
        nxt = load_tile(tb + tstride < t1 ? tb + tstride : t1);
        // ---- scores of the G heads against tokens tb .. tb + 15 ----
        v4f acc = v4f{0.f, 0.f, 0.f, 0.f};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[0], codes_to_bf16(cur.k0.x, cur.k0.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[1], codes_to_bf16(cur.k0.z, cur.k0.w), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[2], codes_to_bf16(cur.k1.x, cur.k1.y), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[3], codes_to_bf16(cur.k1.z, cur.k1.w), acc, 0, 0, 0);
        // 4 x 4 transpose of the row blocks (x[g][r] = row g of register r):
        // swapping the upper halves of registers (0, 2) and (1, 3), then the
        // odd rows of the new register 0 with the even rows of the new
        // register 1, leaves row g of register r holding x[r][g], i.e. head
        // 4 r + g of token tb + n
        // (the elements go through plain scalars: this compiler's bit_cast of
        // an indexed vector element reads element 0)
        float st[R];
        {
            const float x0 = acc[0], x1 = acc[1], x2 = acc[2], x3 = acc[3];
            const auto s02 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x0),
                                                              __builtin_bit_cast(uint32_t, x2), false, false);
            const auto s13 = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x1),
                                                              __builtin_bit_cast(uint32_t, x3), false, false);
            const uint32_t n0 = s02[0], n1 = s13[0];
            const auto s01 = __builtin_amdgcn_permlane16_swap(n0, n1, false, false);
            const uint32_t t0 = s01[0], t1 = s01[1];
            st[0] = __builtin_bit_cast(float, t0);
            if constexpr (R > 1)
                st[1] = __builtin_bit_cast(float, t1);
        }
        const bool tok_ok = tb + n < t1;
        const float kscale = cur.ks * a.scale_log2; // scores in log2 units
        float p[R], alpha[R];
        bool moved = false; // a running max of this lane's heads changed
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float s = tok_ok ? st[r] * kscale : -INFINITY;
            const float mt = row16_fmax(s);                       // finite: token tb is below t1
            const float mnew = mh[r] > mt ? mh[r] : mt;
            alpha[r] = __builtin_amdgcn_exp2f(mh[r] - mnew);      // 0 on the first tile
            p[r] = __builtin_amdgcn_exp2f(s - mnew);              // 0 for masked tokens
            lh[r] = lh[r] * alpha[r] + row16_fsum(p[r]);
            mh[r] = mnew;
            moved = moved || (4 * r + grp < G && alpha[r] != 1.0f);
        }
        // p * vs of each (token, head) and the heads' rescale factors to the wave's LDS
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int h = 4 * r + grp;
            if (h < G) {
                sh.pv[wave][n * G + h] = p[r] * cur.vs;
                if (n == 0)
                    sh.alpha[wave][h] = alpha[r];
            }
        }
        // ---- values: tokens ts + TG u of the tile, dims d0 .. d0 + DPL - 1 ----
        // (LDS writes and reads of one wave complete in order.)  The output
        // is rescaled only on tiles where some head's running max moved: a
        // factor of exactly 1 leaves it unchanged, so skipping it changes no
        // bit, and past the first tiles the max rarely moves
        if (__builtin_amdgcn_ballot_w64(moved)) {
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float al = sh.alpha[wave][h];
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    o[h][e] *= al;
            }
        }
        // (value codes of tokens at or past len read as zeros: their p is 0)
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int t = ts + TG * u;
            float v[DPL];
#pragma unroll
            for (int w = 0; w < DPL / 4; ++w) {
                const f2v lo = __builtin_amdgcn_cvt_pk_f32_fp8(cur.v[u][w], false);
                const f2v hi = __builtin_amdgcn_cvt_pk_f32_fp8(cur.v[u][w], true);
                v[4 * w] = lo.x, v[4 * w + 1] = lo.y, v[4 * w + 2] = hi.x, v[4 * w + 3] = hi.y;
            }
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float pw = sh.pv[wave][t * G + h];
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    o[h][e] = __builtin_fmaf(pw, v[e], o[h][e]);
            }
        }
    }

    // ---- sum the token groups' partials; lanes of group 0 write ----
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
#pragma unroll
            for (int m = LPG; m < 64; m *= 2)
                o[h][e] += __shfl_xor(o[h][e], m);
        }
    // head h's (max, sum) sit in row h % 4, register h / 4, of every lane of that row
    float mrow[G], lrow[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        mrow[h] = __shfl(mh[h / 4], 16 * (h % 4));
        lrow[h] = __shfl(lh[h / 4], 16 * (h % 4));
    }
    if (ts == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            const int64_t bh = b * a.Hq + g * G + h;
            if constexpr (SPLIT) {
                float *pp = a.part + (bh * a.splits + split) * (2 + AD);
                if (n == 0) {
                    pp[0] = mrow[h];
                    pp[1] = lrow[h];
                }
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    pp[2 + d0 + e] = o[h][e];
            } else {
                float r[DPL];
#pragma unroll
                for (int e = 0; e < DPL; ++e)
                    r[e] = lrow[h] > 0.0f ? o[h][e] / lrow[h] : 0.0f;
#pragma unroll
                for (int w = 0; w < DPL / 4; ++w) {
                    if constexpr (OUT_F32) {
                        *(v4f *)((float *)a.out + bh * AD + d0 + 4 * w) =
                            v4f{r[4 * w], r[4 * w + 1], r[4 * w + 2], r[4 * w + 3]};
                    } else {
                        const bf2v p0 = __builtin_convertvector(f2v{r[4 * w], r[4 * w + 1]}, bf2v);
                        const bf2v p1 = __builtin_convertvector(f2v{r[4 * w + 2], r[4 * w + 3]}, bf2v);
                        *(u32x2 *)((__bf16 *)a.out + bh * AD + d0 + 4 * w) =
                            u32x2{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1)};
                    }
                }
            }
        }
    }
}

// Merge of the splits of one (sequence, query head): one wave each, lane l
// takes dims 2 l and 2 l + 1; the splits are added in split order.  Lane s
// loads split s's (max, sum) (splits <= 64, checked at launch), so those loads are in flight
// together; the wave's max is a butterfly, lane s forms split s's factor and
// every lane takes the factors in split order by lane reads, with the splits'
// outputs loaded four splits ahead.  The sums are those of a lane that loads
// and weighs the splits one after another, bit for bit.
template <bool OUT_F32>
__global__ __launch_bounds__(64) void kv_attn_combine_kernel(const float *part, int splits, void *out)
{
    const int64_t bh = blockIdx.x;
    const int lane = threadIdx.x;
    const float *pp = part + bh * splits * (2 + AD);
    const float ms = lane < splits ? pp[lane * (2 + AD)] : -INFINITY;
    const float ls = lane < splits ? pp[lane * (2 + AD) + 1] : 0.0f;
    float M = ms;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float t = __shfl_xor(M, o);
        M = M > t ? M : t;
    }
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    if (M != -INFINITY) { // (uniform: every lane holds the wave's max)
        const float fs = __builtin_amdgcn_exp2f(ms - M); // split `lane`'s factor (0 past the splits)
        int s = 0;
        for (; s + 4 <= splits; s += 4) {
            float a[4], b[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a[j] = pp[(s + j) * (2 + AD) + 2 + 2 * lane];
                b[j] = pp[(s + j) * (2 + AD) + 3 + 2 * lane];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float f = __shfl(fs, s + j), l = __shfl(ls, s + j);
                L = __builtin_fmaf(f, l, L);
                o0 = __builtin_fmaf(f, a[j], o0);
                o1 = __builtin_fmaf(f, b[j], o1);
            }
        }
        for (; s < splits; ++s) {
            const float f = __shfl(fs, s), l = __shfl(ls, s);
            L = __builtin_fmaf(f, l, L);
            o0 = __builtin_fmaf(f, pp[s * (2 + AD) + 2 + 2 * lane], o0);
            o1 = __builtin_fmaf(f, pp[s * (2 + AD) + 3 + 2 * lane], o1);
        }
    }
    const float r0 = L > 0.0f ? o0 / L : 0.0f, r1 = L > 0.0f ? o1 / L : 0.0f;
    if constexpr (OUT_F32) {
        *(f2v *)((float *)out + bh * AD + 2 * lane) = f2v{r0, r1};
    } else {
        *(bf2v *)((__bf16 *)out + bh * AD + 2 * lane) = __builtin_convertvector(f2v{r0, r1}, bf2v);
    }
}

// Splits per sequence: enough workgroups (of up to 8 key/value heads each)
// to give every CU two, each split at least 256 tokens (rounded so that the
// splits' shares are whole 16-token tiles).
static void attn_plan(int64_t B, int64_t T, int64_t Hkv, int &splits)
{
    const int64_t groups = B * ((Hkv + ATT_WAVES - 1) / ATT_WAVES);
    int64_t s = (512 + groups - 1) / groups;
    const int64_t smax = (T + 255) / 256;
    s = s < smax ? s : smax;
    s = s < 1 ? 1 : (s > 64 ? 64 : s);
    int64_t c = (T + s - 1) / s;
    c = (c + 15) / 16 * 16;
    s = (T + c - 1) / c;
    splits = (int)(s < 1 ? 1 : s);
}

size_t kv_attention_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv)
{
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0)
        return 0;
    int splits;
    attn_plan(B, T, Hkv, splits);
    return splits > 1 ? (size_t)B * (size_t)Hq * (size_t)splits * (2 + AD) * sizeof(float) : 0;
}

template <int G>
static hipError_t run_attn(const AttnArgs &a, bool out_f32, hipStream_t stream)
{
    const dim3 grid((unsigned)(a.B * ((a.Hkv + ATT_WAVES - 1) / ATT_WAVES)), (unsigned)a.splits),
        block(ATT_WAVES * 64);
    if (a.splits > 64)
        return hipErrorInvalidValue; // (attn_plan caps the splits at 64: one per lane of the merge)
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
    attn_plan(B, T, Hkv, a.splits);
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
