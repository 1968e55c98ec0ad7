// fp8bs_device.hpp -- device helpers shared by the gfx950 kernels.
//
// Quantization rule (the article "NVIDIA NeMo RL achieves 48% speedup with
// end-to-end FP8 precision training", section "Technical breakthrough":
// block-wise E4M3 with 1x128 / 128x128 blocks; closing section: optional
// power-of-2 scaling factors):
//   amax = max |x| over the block (exact);
//   EXACT: s = RN_fp32(amax / 448);  POW2: s = 2^k, least k with amax <= 448*2^k;
//   an all-zero block takes s = 1;
//   q = E4M3_sat_RNE(RN_fp32(x / s)), sign of x kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---- bf16 -----------------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Largest |bf16| magnitude payload among the 8 values of a 16-byte chunk,
// returned as a 16-bit magnitude payload in the low half (finite values
// order like their payloads once the sign bit is cleared).
__device__ __forceinline__ uint32_t chunk_max_mag(u32x4 v)
{
    uint32_t a = v.x & 0x7fff7fffu, b = v.y & 0x7fff7fffu, c = v.z & 0x7fff7fffu, d = v.w & 0x7fff7fffu;
    typedef unsigned short us2 __attribute__((ext_vector_type(2)));
    us2 m = __builtin_elementwise_max(__builtin_elementwise_max(__builtin_bit_cast(us2, a), __builtin_bit_cast(us2, b)),
                                      __builtin_elementwise_max(__builtin_bit_cast(us2, c), __builtin_bit_cast(us2, d)));
    uint32_t lo = m.x, hi = m.y;
    return lo > hi ? lo : hi;
}

// Max over the 16 lanes of a DPP row (lanes 16r .. 16r+15); every lane of the
// row receives the result.  All 16 lanes must be active.
__device__ __forceinline__ uint32_t row16_max(uint32_t v)
{
    uint32_t t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm [1,0,3,2]
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm [2,3,0,1]
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false); // row_half_mirror
    v = v > t ? v : t;
    t = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false); // row_mirror
    v = v > t ? v : t;
    return v;
}

// ---- scales ------------------------------------------------------------------

enum { SCALE_EXACT = 0, SCALE_POW2 = 1 };

// amax as fp32 from its bf16 magnitude payload.
__device__ __forceinline__ float amax_value(uint32_t mag16) { return __uint_as_float(mag16 << 16); }

// Exponent k of the POW2 scale: the least integer with amax <= 448 * 2^k.
// amax = 2^E * m, m in [1, 2); 448 = 1.75 * 2^8, so k = E - 8 + (m > 1.75).
// Integer-exact for every positive finite amax, subnormals included.
__device__ __forceinline__ int pow2_exponent(float amax)
{
    uint32_t u = __float_as_uint(amax);
    uint32_t ef = u >> 23, mf = u & 0x7fffffu;
    if (ef != 0)
        return (int)ef - 127 - 8 + (mf > 0x600000u ? 1 : 0);
    // subnormal amax = mf * 2^-149 with highest set bit p: E = p - 149, m = mf / 2^p
    int p = 31 - __builtin_clz(mf);
    uint32_t frac = (mf << (23 - p)) & 0x7fffffu; // mantissa field of the normalized m
    return p - 149 - 8 + (frac > 0x600000u ? 1 : 0);
}

// 2^k as fp32 (k >= -149), exact.
__device__ __forceinline__ float exp2_int(int k)
{
    return k >= -126 ? __uint_as_float((uint32_t)(k + 127) << 23) : __uint_as_float(1u << (k + 149));
}

template <int MODE>
__device__ __forceinline__ float block_scale(float amax)
{
    if (!(amax > 0.0f))
        return 1.0f;
    if (MODE == SCALE_POW2)
        return exp2_int(pow2_exponent(amax));
    return amax / 448.0f; // IEEE, correctly rounded (HIP default, denormals kept)
}

// ---- correctly rounded x / s ---------------------------------------------
//
// The quotient must be RN_fp32(x / s) bit for bit.  A multiply by RN(1/s)
// is NOT that (it changes about 1 code in 16000), so the divider below runs
// the Newton-Raphson refinement that the compiler's own IEEE division uses,
// without its range-scaling and fix-up steps, which act only on operands
// outside the window this library feeds it:
//   - s is a normal number in [2^-80, 2^126): every EXACT scale of a block
//     whose amax is at least 448 * 2^-80 (the kernels fall back to the full
//     IEEE division for smaller blocks);
//   - |x| <= amax, so |x / s| <= 448 (no overflow), and when |x| is so small
//     that the refinement's residuals leave the normal range (|x| < 2^-100),
//     |x / s| < 2^-20, whose code is 0 whatever the last bits are.
// The sign of a zero quotient is restored from x (the residual steps turn
// -0 into +0).  Exhaustive tests over every bf16 (x, amax) pair check this
// against the oracle's IEEE division.
struct Divider {
    float s, r;
    __device__ __forceinline__ void init(float s_)
    {
        s = s_;
        float r0 = __builtin_amdgcn_rcpf(s_);
        float e0 = __builtin_fmaf(-s_, r0, 1.0f);
        r = __builtin_fmaf(e0, r0, r0);
    }
    __device__ __forceinline__ float div(float x) const
    {
        float q0 = x * r;
        float e1 = __builtin_fmaf(-s, q0, x);
        float q1 = __builtin_fmaf(e1, r, q0);
        float e2 = __builtin_fmaf(-s, q1, x);
        float q = __builtin_fmaf(e2, r, q1);
        return __builtin_copysignf(q, x);
    }
};

// Blocks whose EXACT scale is outside the Divider window take IEEE division.
__device__ __forceinline__ bool divider_ok(float s) { return s >= 0x1p-80f && s < 0x1p126f; }

// ---- E4M3 -------------------------------------------------------------------
//
// v_cvt_pk_fp8_f32 on gfx950 converts two fp32 values to OCP E4M3 with
// round-to-nearest-even; quotients here never exceed 448 * (1 + 2^-23), which
// rounds to 448, so no saturation case reaches it.  `word` selects the low
// (false) or high (true) 16 bits of `old` to replace.
template <bool WORD>
__device__ __forceinline__ uint32_t cvt_pk_e4m3(float a, float b, uint32_t old)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, WORD);
}

// Four quotients -> one dword of codes (byte i = code of q_i).
__device__ __forceinline__ uint32_t pack4_e4m3(float q0, float q1, float q2, float q3)
{
    uint32_t w = cvt_pk_e4m3<false>(q0, q1, 0u);
    return cvt_pk_e4m3<true>(q2, q3, w);
}

// ---- one block's encoder (shared by the quantizers and the GEMM that
// quantizes its activations itself) ------------------------------------------

// Per-block quotient state: the fast path (Newton division / exact multiply)
// or, for the rare blocks outside its window, IEEE division.
template <int MODE>
struct BlockQuant {
    float s;    // dequantization scale
    float inv;  // POW2: 2^-k
    Divider d;  // EXACT
    bool fast;

    __device__ __forceinline__ void init(float amax)
    {
        s = block_scale<MODE>(amax);
        if (MODE == SCALE_POW2) {
            // 2^-k is a normal fp32 for k in [-126, 127]; k never exceeds 120
            // for finite bf16 amax, so only tiny blocks miss the fast path.
            int k = (amax > 0.0f) ? pow2_exponent(amax) : 0;
            fast = k >= -126;
            inv = fast ? exp2_int(-k) : 1.0f;
        } else {
            fast = divider_ok(s);
            d.init(fast ? s : 1.0f);
        }
    }
    __device__ __forceinline__ float q_fast(float x) const
    {
        if (MODE == SCALE_POW2)
            return x * inv; // x * 2^-k == x / s exactly, rounded once (subnormals kept)
        return d.div(x);
    }
};

// 4 values (bf16 values widened to fp32) -> one dword of codes.
template <int MODE>
__device__ __forceinline__ uint32_t quant4(float x0, float x1, float x2, float x3, const BlockQuant<MODE> &bq)
{
    if (bq.fast)
        return pack4_e4m3(bq.q_fast(x0), bq.q_fast(x1), bq.q_fast(x2), bq.q_fast(x3));
    const float s = bq.s;
    return pack4_e4m3(x0 / s, x1 / s, x2 / s, x3 / s);
}

// The IEEE-division path of quant4 out of line, for callers that inline many
// quant4 calls on a path that is rarely taken (the GEMM epilogue): it keeps
// their code, and the instruction cache it occupies, small.
__device__ __noinline__ uint32_t quant4_ieee(float x0, float x1, float x2, float x3, float s)
{
    return pack4_e4m3(x0 / s, x1 / s, x2 / s, x3 / s);
}

// quant4's fast path alone (the caller has checked bq.fast).
template <int MODE>
__device__ __forceinline__ uint32_t quant4_fast(float x0, float x1, float x2, float x3, const BlockQuant<MODE> &bq)
{
    return pack4_e4m3(bq.q_fast(x0), bq.q_fast(x1), bq.q_fast(x2), bq.q_fast(x3));
}

// 8 bf16 values (one 16-byte chunk) -> 8 codes.
template <int MODE>
__device__ __forceinline__ u32x2 quant_chunk(u32x4 v, const BlockQuant<MODE> &bq)
{
    u32x2 out;
    out.x = quant4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y), bq);
    out.y = quant4(bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w), bq);
    return out;
}

} // namespace fp8bs
