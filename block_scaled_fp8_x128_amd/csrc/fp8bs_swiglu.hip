// fp8bs_swiglu.hip -- the MLP's gated activation fused with the 1x128
// activation quantizer of the down projection's input.
//
// The article "NVIDIA NeMo RL achieves 48% speedup with end-to-end FP8
// precision training", section "Technical breakthrough", keeps non-linear
// functions in BF16 and runs the linear layers in FP8; section "Real-world
// performance gains" names quantization kernel overhead as part of the gap to
// the 2x peak.  Between the gate+up and the down projection of its MLP models
// the gated activation h = silu(g) * u (a bf16 tensor) is followed by the 1x128
// quantizer; this kernel does both in one pass over the gate+up output:
//
//   gu [M, 2F] bf16, gate columns 0..F-1, up columns F..2F-1 of each row
//   h[m, f]  = RN_bf16((g * sigma(g)) * u),  sigma(g) = 1 / (1 + exp(-g)),
//              the value the fp64 evaluation of that expression rounds to
//   hq, hs   = quant_act_1x128(h): codes [M, F], scales [M, F/128]
//
// so it reads 4 bytes and writes 1 + 4/128 bytes per element of h, against
// 4 + 2 (h written) + 2 + 1 + 4/128 for the activation followed by the
// quantizer.  The block layout is the activation quantizer's: each 16-lane
// DPP row owns one 1x128 block of h, one 8-value chunk per lane (16 bytes of
// gate and 16 of up).
//
// Precision.  h is computed in fp32 (the hardware base-2 exponential of an
// exact argument with a first-order correction, the hardware reciprocal, an
// exact product g * u and one more product: about 5 units in the last place
// of fp32 at most by analysis, 3.1 the largest seen over every bf16 gate
// value) and rounded to bf16 from there by the hardware conversion.  That
// rounding agrees with the rounding of the fp64 value unless the fp32 value
// lies within a few fp32 units of a bf16 rounding midpoint; such elements
// (low 16 bits of the fp32 pattern within 16 of 0x8000: over three times the
// bound), and every element whose operands or result leave the range where
// the fp32 error bound holds (g < -64, h zero, subnormal, infinite or NaN),
// are recomputed in fp64 and rounded from there.  About 0.05% of elements
// take the fp64 path; the window is kept narrow because a wave runs the fp64
// path for an element slot whenever one of its lanes needs it.
#include "fp8bs_device.hpp"
#include "fp8bs_internal.hpp"

namespace fp8bs {

constexpr int SG_UNROLL = 2;
constexpr int SG_THREADS = 256;
constexpr int SG_BLOCKS_PER_WG = (SG_THREADS / 64) * 4 * SG_UNROLL;

// Nearest bf16 payload (ties to even) of a double.
__device__ __noinline__ uint32_t bf16_of_double(double v)
{
    const uint32_t sign = (__double_as_longlong(v) < 0) ? 0x8000u : 0u;
    const double a = fabs(v);
    if (a != a)
        return sign | 0x7FC0u;
    if (a == 0.0)
        return sign;
    if (a > 1.0e39) // far beyond the largest finite bf16 (about 3.39e38)
        return sign | 0x7F80u;
    const int e = ilogb(a);                     // a in [2^e, 2^(e+1))
    const int qe = (e >= -126 ? e : -126) - 7;  // spacing of bf16 values there
    const double r = ldexp(rint(ldexp(a, -qe)), qe);
    if (r >= 0x1p128)
        return sign | 0x7F80u;
    return sign | (__float_as_uint((float)r) >> 16); // exact: r has at most 8 significant bits
}

__device__ __noinline__ uint32_t swiglu_fp64(float g, float u)
{
    const double gd = (double)g, ud = (double)u;
    const double sig = 1.0 / (1.0 + exp(-gd));
    return bf16_of_double((gd * sig) * ud);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// 1 + exp(-g) for g >= -64.  exp(-g) = 2^(-g log2 e) with log2 e split as
// C1 + C2, C1 holding 16 significant bits: th = -g C1 is then exact in fp32
// (g has 8), 2^th comes from the hardware base-2 exponential, and
// 2^(-g C2) = 1 + t with t = -g C2 ln 2, |t| < 3.2e-4; the next term, t^2 / 2
// (below 2^-24), is left out.  1 + exp(-g) = fma(2^th, 1 + t, 1).
__device__ __forceinline__ float one_plus_exp_neg(float g)
{
    constexpr float C1 = 1.44268798828125f;           // 47274 / 32768
    constexpr float C2LN2 = 4.888495152129525e-6f;    // (log2(e) - C1) * ln 2
    const float e = __builtin_amdgcn_exp2f(-g * C1);
    return __builtin_fmaf(e, __builtin_fmaf(-g, C2LN2, 1.0f), 1.0f);
}

// One element on the fp32 path: h, and whether its bf16 rounding is sure.
// When h is a normal fp32, so is g * u (|g * u| >= |h|), and g * u is then
// exact (two 8-bit significands); the relative error of h is that of
// sigma(g) plus one rounding, below about 5 units in the last place (the
// exponential about 2, the reciprocal 1).  Elements within 16 units of a bf16
// rounding midpoint, or outside the range where that bound holds (g < -64, h
// zero, subnormal, infinite or NaN), are flagged for fp64.  The tests are
// combined without short-circuit branches so that the fp32 path stays
// straight-line.
__device__ __forceinline__ float swiglu_fast(float g, float u, bool &ok)
{
    const float sig = __builtin_amdgcn_rcpf(one_plus_exp_neg(g));
    const float h = (g * u) * sig;
    const uint32_t b = __float_as_uint(h);
    constexpr int NORMAL = 0x008 | 0x100; // negative normal | positive normal
    ok = (g >= -64.0f) & __builtin_amdgcn_classf(h, NORMAL) & (((b & 0xFFFFu) - (0x8000u - 16u)) > 32u);
    return h;
}

// Two fp32 values -> their bf16 payloads (round to nearest even), packed.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi)
{
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// 8 gate and 8 up values (one 16-byte chunk each) -> 8 h payloads, packed.
// The flagged elements are recomputed in fp64 afterwards, one branch per
// element that the whole wave skips unless one of its lanes needs it.
__device__ __forceinline__ u32x4 swiglu_chunk(u32x4 g, u32x4 u)
{
    const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
    uint32_t hw[4];
    bool ok[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const float lo = swiglu_fast(bf16_lo(gw[d]), bf16_lo(uw[d]), ok[2 * d]);
        const float hi = swiglu_fast(bf16_hi(gw[d]), bf16_hi(uw[d]), ok[2 * d + 1]);
        hw[d] = pack_bf16(lo, hi);
    }
    bool all = true;
#pragma unroll
    for (int k = 0; k < 8; ++k)
        all &= ok[k];
    if (__builtin_expect(!all, 0)) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (!ok[k]) {
                const int d = k / 2;
                const uint32_t p = (k & 1) ? swiglu_fp64(bf16_hi(gw[d]), bf16_hi(uw[d]))
                                           : swiglu_fp64(bf16_lo(gw[d]), bf16_lo(uw[d]));
                hw[d] = (k & 1) ? ((hw[d] & 0xFFFFu) | (p << 16)) : ((hw[d] & 0xFFFF0000u) | p);
            }
        }
    }
    return u32x4{hw[0], hw[1], hw[2], hw[3]};
}

template <int MODE>
__global__ __launch_bounds__(SG_THREADS) void swiglu_quant_kernel(const uint16_t *__restrict__ gu,
                                                                 u32x2 *__restrict__ q, float *__restrict__ s,
                                                                 uint32_t nblocks, uint32_t FB)
{
    const int lane = threadIdx.x & 63;
    const int slot = lane >> 4; // block slot of this DPP row
    const int c = lane & 15;    // 8-value chunk within the block
    const uint32_t wave = blockIdx.x * (SG_THREADS / 64) + (threadIdx.x >> 6);
    const uint32_t b0 = wave * (4 * SG_UNROLL) + slot;
    const int64_t F = (int64_t)FB * 128;

    u32x4 gv[SG_UNROLL], uv[SG_UNROLL];
#pragma unroll
    for (int j = 0; j < SG_UNROLL; ++j) {
        const uint32_t b = b0 + 4 * j;
        if (b < nblocks) {
            const uint32_t m = b / FB, fb = b - m * FB;
            const uint16_t *p = gu + (int64_t)m * 2 * F + (int64_t)fb * 128 + 8 * c;
            gv[j] = __builtin_nontemporal_load((const u32x4 *)p);
            uv[j] = __builtin_nontemporal_load((const u32x4 *)(p + F));
        } else {
            gv[j] = u32x4{0u, 0u, 0u, 0u};
            uv[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int j = 0; j < SG_UNROLL; ++j) {
        const uint32_t b = b0 + 4 * j;
        const u32x4 h = swiglu_chunk(gv[j], uv[j]);
        // every lane takes part in the DPP reduction (blocks past the end hold zeros)
        const float amax = amax_value(row16_max(chunk_max_mag(h)));
        BlockQuant<MODE> bq;
        bq.init(amax);
        const u32x2 codes = quant_chunk<MODE>(h, bq);
        if (b < nblocks) {
            q[(int64_t)b * 16 + c] = codes; // (cached: the down projection's operand next)
            if (c == 0)
                s[b] = bq.s;
        }
    }
}

hipError_t launch_swiglu_quant(const void *gu, int64_t M, int64_t F, void *hq, float *hs, int mode,
                               hipStream_t stream)
{
    const int64_t nblocks = M * (F / 128);
    if (nblocks == 0)
        return hipSuccess;
    const int64_t grid = (nblocks + SG_BLOCKS_PER_WG - 1) / SG_BLOCKS_PER_WG;
    if (mode == SCALE_POW2)
        return launch(swiglu_quant_kernel<SCALE_POW2>, dim3((unsigned)grid), dim3(SG_THREADS), 0, stream,
                      (const uint16_t *)gu, (u32x2 *)hq, hs, (uint32_t)nblocks, (uint32_t)(F / 128));
    return launch(swiglu_quant_kernel<SCALE_EXACT>, dim3((unsigned)grid), dim3(SG_THREADS), 0, stream,
                  (const uint16_t *)gu, (u32x2 *)hq, hs, (uint32_t)nblocks, (uint32_t)(F / 128));
}

} // namespace fp8bs
