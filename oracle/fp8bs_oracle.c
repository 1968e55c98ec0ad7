/*
 * fp8bs_oracle.c -- plain CPU oracle of the block-wise FP8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark load this file's library.  It shares no code,
 * header, table or constant with the GPU library, and the GPU library never
 * calls it.
 *
 * Source of the method: the article "NVIDIA NeMo RL achieves 48% speedup with
 * end-to-end FP8 precision training" (Jessie A Ellis, Apr 20 2026), published
 * in three translations (mexc.co/hi-IN/news/1041474,
 * alookzone.com/bn-BD/news/1041474, hotbookzone.com/ar-AE/news/1041474).  Its
 * section "Technical breakthrough" states that the recipe quantizes block-wise
 * to FP8 in the E4M3 format, with 128x128 blocks for weights and 1x128 blocks
 * for activations, and that linear layers then run FP8 math.  Its section
 * "Real-world performance gains" states that the quantization scales are
 * recalibrated after every training step.  Its closing section names
 * power-of-2 scaling factors as an option.  Everything else below -- the
 * amax/448 scale rule, saturating round-to-nearest-even, fp32 scales, the
 * per-128-K scale application, the MoE grouped form -- is the project's
 * statement of the method, since the article is silent on it; each such
 * reading is marked READING.
 *
 * Every result here is computed from its definition, one element at a time:
 *   - E4M3 codes by search over the 127 non-negative finite magnitudes;
 *   - fp32 scales and quotients by single IEEE fp32 operations;
 *   - each 128-wide block of a GEMM dot product exactly, in int64, then the
 *     scale products and the sum over blocks in fp64.
 * Build: gcc -O2 -fopenmp -ffp-contract=off (no fast-math: the fp32 division
 * below must be the correctly rounded IEEE one, with subnormals kept).
 *
 * Pins (tests that tie each function to something other than itself):
 *   e4m3_decode/encode : hand values of the format definition, all 256 codes,
 *                        midpoint ties, torch's float8_e4m3fn cast;
 *   block_scale        : amax element -> code 0x7E for every bf16 amax,
 *                        power-of-two bounds, zero blocks;
 *   quant_*            : sign / power-of-two / permutation / transposition
 *                        invariants, error bound, brute force on tiny shapes,
 *                        torch's fp32 division + fp8 cast;
 *   gemm, grouped_gemm : numpy fp64 matmul of the dequantized operands,
 *                        integer special cases, per-expert decomposition;
 *   gemm_1x128         : numpy fp64 matmul of the dequantized operands (row
 *                        scales on both), the block-scaled gemm where the row
 *                        scales are constant over 128 rows, integer case;
 *   bf16_from_double   : integer rounding of fp32 bit patterns, torch's
 *                        float32 -> bfloat16 cast, hand midpoints, subnormal
 *                        and overflow boundaries;
 *   swiglu_*           : 50-digit decimal evaluation rounded to bf16 by exact
 *                        rational arithmetic, closed-form special cases.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- E4M3 (OCP 8-bit floating point, "E4M3FN": bias 7, no infinities,
 *      NaN = S.1111.111, largest finite magnitude 448) ---------------------- */

/* Value of one E4M3 code, exactly, as a double.  Code bits: s eeee mmm.
 * e == 0: subnormal, m * 2^-9.  e >= 1: 2^(e-7) * (1 + m/8).  e == 15 and
 * m == 7: NaN. */
double oracle_e4m3_decode(uint32_t code)
{
    uint32_t s = (code >> 7) & 1u, e = (code >> 3) & 15u, m = code & 7u;
    double mag;
    if (e == 15u && m == 7u)
        return NAN;
    if (e == 0u)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);
    return s ? -mag : mag;
}

/* Saturating round-to-nearest-even encoding of a finite fp32 value.
 * READING: the magnitude goes to the nearest of the 127 non-negative finite
 * E4M3 magnitudes (codes 0x00..0x7E), a tie to the code whose mantissa LSB
 * (= code bit 0) is 0; magnitudes at or above 448 give 0x7E (saturation).
 * The sign bit is copied from the input, so -0 and small negatives give 0x80.
 * NaN input gives 0x7F with the sign (out of the quantizer's contract). */
uint32_t oracle_e4m3_encode(float v)
{
    uint32_t sign = signbit(v) ? 0x80u : 0u;
    double a, lo_v, hi_v, mid;
    int lo, hi;
    if (isnan(v))
        return sign | 0x7Fu;
    a = fabs((double)v);
    if (a >= 448.0)
        return sign | 0x7Eu;
    /* largest code lo in [0, 126] with decode(lo) <= a (decode(0) = 0 <= a) */
    lo = 0;
    hi = 126;
    while (lo < hi) {
        int mid_c = (lo + hi + 1) / 2;
        if (oracle_e4m3_decode((uint32_t)mid_c) <= a)
            lo = mid_c;
        else
            hi = mid_c - 1;
    }
    /* a < 448 = decode(126), so lo <= 125 and decode(lo) <= a < decode(lo+1) */
    lo_v = oracle_e4m3_decode((uint32_t)lo);
    hi_v = oracle_e4m3_decode((uint32_t)lo + 1u);
    mid = 0.5 * (lo_v + hi_v); /* exact: both have at most 4 significant bits */
    if (a < mid)
        return sign | (uint32_t)lo;
    if (a > mid)
        return sign | (uint32_t)(lo + 1);
    return sign | (uint32_t)((lo & 1) ? lo + 1 : lo);
}

void oracle_e4m3_encode_array(const float *v, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = (uint8_t)oracle_e4m3_encode(v[i]);
}

void oracle_e4m3_decode_array(const uint8_t *c, int64_t n, double *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_decode(c[i]);
}

/* bf16 is the upper 16 bits of an fp32 word. */
static float bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* ---- block scale --------------------------------------------------------- */

enum { ORACLE_SCALE_EXACT = 0, ORACLE_SCALE_POW2 = 1 };

/* Dequantization scale s of a block whose largest magnitude is amax
 * (x ~= decode(q) * s).
 * EXACT (READING): s = amax / 448, one correctly rounded fp32 division, so the
 *   block's largest element maps to +-448.
 * POW2 (READING of the article's "power-of-2 scaling factors"): s = 2^k with
 *   k the least integer such that amax <= 448 * 2^k, decided by exact
 *   comparison; rounding the scale up never clips.
 * READING: an all-zero block (amax = 0) takes s = 1. */
float oracle_block_scale(float amax, int mode)
{
    if (!(amax > 0.0f))
        return 1.0f;
    if (mode == ORACLE_SCALE_POW2) {
        int k;
        double a = (double)amax;
        (void)frexp(a / 448.0, &k); /* a/448 in [2^(k-1), 2^k) up to rounding */
        while (a > 448.0 * ldexp(1.0, k))
            ++k;
        while (a <= 448.0 * ldexp(1.0, k - 1))
            --k;
        return ldexpf(1.0f, k);
    }
    return amax / 448.0f;
}

/* Code of one element: q = E4M3( RN_fp32(x / s) ).  READING: the quotient is
 * the correctly rounded fp32 division (the precision of the fp32 scale), then
 * encoded; the two roundings are the definition. */
static uint32_t quant_element(float x, float s)
{
    volatile float q = x / s;
    return oracle_e4m3_encode(q);
}

/* Activation quantizer, 1x128 blocks along K.
 * x: bf16 payloads [M, K] row-major.  q: codes [M, K].  s: fp32 [M, K/128].
 * Block (m, kb) = x[m, 128 kb .. 128 kb + 127].  K must be a multiple of 128. */
static void quant_act_block(const uint16_t *xb, uint8_t *qb, float *sb, int mode)
{
    float amax = 0.0f, sc;
    int k;
    for (k = 0; k < 128; ++k) {
        float a = fabsf(bf16_value(xb[k]));
        if (a > amax)
            amax = a;
    }
    sc = oracle_block_scale(amax, mode);
    for (k = 0; k < 128; ++k)
        qb[k] = (uint8_t)quant_element(bf16_value(xb[k]), sc);
    *sb = sc;
}

void oracle_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, uint8_t *q, float *s, int mode)
{
    int64_t KB = K / 128, b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < M * KB; ++b) {
        int64_t m = b / KB, kb = b % KB;
        quant_act_block(x + m * K + kb * 128, q + m * K + kb * 128, s + m * KB + kb, mode);
    }
}

/* ---- the gated activation between the MLP projections ------------------- */

/* Nearest bf16 (ties to the even payload) of a double, as a bf16 payload.
 * bf16 keeps 8 significant bits over fp32's exponent range: the spacing of
 * the values in [2^e, 2^(e+1)) is 2^(e-7) for e >= -126, and 2^-133 below
 * (subnormals).  Rounding past the largest finite value gives infinity. */
uint16_t oracle_bf16_from_double(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v), r;
    float f;
    uint32_t u;
    int e, qe;
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    if (a == 0.0)
        return sign;
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    (void)frexp(a, &e); /* a in [2^(e-1), 2^e) */
    qe = (e - 1 >= -126) ? (e - 1) - 7 : -133;
    r = nearbyint(ldexp(a, -qe)); /* the default rounding mode: nearest, ties to even */
    r = ldexp(r, qe);
    if (r >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    f = (float)r; /* exact: r has at most 8 significant bits */
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(sign | (u >> 16));
}

/* SiLU-gated linear unit of the MLP, from the gate+up projection's output.
 * READING: the article's MLP models (Llama 3.1 8B, Qwen3-30B; opening and
 * "Real-world performance gains" sections) gate their MLP with
 * h = silu(g) * u, silu(g) = g * sigma(g), sigma the logistic function; the
 * article names no activation.  Its section "Technical breakthrough" keeps
 * non-linear functions in BF16, so h is a bf16 tensor: the value computed in
 * fp64 as (g * sigma(g)) * u with sigma(g) = 1 / (1 + exp(-g)), rounded once
 * to bf16.  READING: gu [M, 2F] row-major holds the gate values in columns
 * 0 .. F-1 and the up values in columns F .. 2F-1 of each row.
 * h: bf16 payloads [M, F]. */
static uint16_t swiglu_element(uint16_t g_bf16, uint16_t u_bf16)
{
    double g = (double)bf16_value(g_bf16), u = (double)bf16_value(u_bf16);
    double sig = 1.0 / (1.0 + exp(-g));
    return oracle_bf16_from_double((g * sig) * u);
}

void oracle_swiglu_bf16(const uint16_t *gu, int64_t M, int64_t F, uint16_t *h)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M * F; ++i) {
        int64_t m = i / F, f = i % F;
        h[i] = swiglu_element(gu[m * 2 * F + f], gu[m * 2 * F + F + f]);
    }
}

/* The gated activation, then the 1x128 activation quantizer of the down
 * projection's input: q [M, F], s [M, F/128].  F must be a multiple of 128. */
void oracle_swiglu_quant_1x128(const uint16_t *gu, int64_t M, int64_t F, uint8_t *q, float *s, int mode)
{
    int64_t FB = F / 128, b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < M * FB; ++b) {
        int64_t m = b / FB, fb = b % FB, k;
        uint16_t h[128];
        for (k = 0; k < 128; ++k)
            h[k] = swiglu_element(gu[m * 2 * F + fb * 128 + k], gu[m * 2 * F + F + fb * 128 + k]);
        quant_act_block(h, q + m * F + fb * 128, s + b, mode);
    }
}

/* Weight quantizer, 128x128 blocks.
 * w: bf16 payloads [N, K] row-major.  q: codes [N, K].  s: fp32 [N/128, K/128].
 * Block (nb, kb) = w[128 nb .. 128 nb + 127, 128 kb .. 128 kb + 127].
 * N and K must be multiples of 128. */
void oracle_quant_w_128x128(const uint16_t *w, int64_t N, int64_t K, uint8_t *q, float *s, int mode)
{
    int64_t NB = N / 128, KB = K / 128, b;
#pragma omp parallel for schedule(static)
    for (b = 0; b < NB * KB; ++b) {
        int64_t nb = b / KB, kb = b % KB, r, c;
        float amax = 0.0f, sc;
        for (r = 0; r < 128; ++r)
            for (c = 0; c < 128; ++c) {
                float a = fabsf(bf16_value(w[(nb * 128 + r) * K + kb * 128 + c]));
                if (a > amax)
                    amax = a;
            }
        sc = oracle_block_scale(amax, mode);
        for (r = 0; r < 128; ++r)
            for (c = 0; c < 128; ++c) {
                int64_t i = (nb * 128 + r) * K + kb * 128 + c;
                q[i] = (uint8_t)quant_element(bf16_value(w[i]), sc);
            }
        s[nb * KB + kb] = sc;
    }
}

/* ---- block-scaled GEMM ----------------------------------------------------- */

/* decode(c) * 2^9 is an integer for every finite code (|.| <= 229376). */
static int e4m3_times_512(uint32_t c, int *is_nan)
{
    double d = oracle_e4m3_decode(c);
    if (isnan(d)) {
        *is_nan = 1;
        return 0;
    }
    return (int)ldexp(d, 9);
}

/* One output element:
 *   Y[m, n] = sum over kb of (xs[m, kb] * ws[n/128, kb]) * P[m, n, kb],
 *   P[m, n, kb] = sum over k in block kb of decode(xq[m, k]) * decode(wq[n, k]),
 * with P exact (int64 of the codes times 2^9 each) and the rest in fp64,
 * blocks taken in ascending kb.  READING: the article says only that linear
 * layers run FP8 math; the per-128-K application of the product of the two
 * fp32 scales is the project's statement of the GEMM. */
static double gemm_element_g(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                             int64_t K, int64_t m, int64_t n, int64_t ws_row)
{
    int64_t KB = K / 128, kb, k;
    double y = 0.0;
    int nan = 0;
    for (kb = 0; kb < KB; ++kb) {
        int64_t p = 0;
        for (k = kb * 128; k < kb * 128 + 128; ++k)
            p += (int64_t)e4m3_times_512(xq[m * K + k], &nan) * (int64_t)e4m3_times_512(wq[n * K + k], &nan);
        y += ((double)xs[m * KB + kb] * (double)ws[ws_row * KB + kb]) * ldexp((double)p, -18);
    }
    return nan ? NAN : y;
}

/* Weight scales per 128x128 block: row n of wq takes the scales of block row n/128. */
static double gemm_element(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                           int64_t K, int64_t m, int64_t n)
{
    return gemm_element_g(xq, xs, wq, ws, K, m, n, n / 128);
}

/* Y = Xq Wq^T with block scales.  xq [M, K], xs [M, K/128], wq [N, K],
 * ws [N/128, K/128], y fp64 [M, N], all row-major. */
void oracle_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                 int64_t M, int64_t N, int64_t K, double *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M * N; ++i)
        y[i] = gemm_element(xq, xs, wq, ws, K, i / N, i % N);
}

/* The same GEMM at chosen output positions (rows[i], cols[i]) only. */
void oracle_gemm_sampled(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                         int64_t M, int64_t N, int64_t K, const int64_t *rows, const int64_t *cols,
                         int64_t count, double *y)
{
    int64_t i;
    (void)M;
    (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i)
        y[i] = gemm_element(xq, xs, wq, ws, K, rows[i], cols[i]);
}

/* The same product with 1x128 scales on both operands: ws [N, K/128] holds one
 * scale per row of wq and K block (the weight gradient dW = dY^T X, both of
 * whose operands are activation-like and quantized along the tokens).
 * READING: the article says its recipe also runs in training but not how the
 * backward products are blocked; the 1x128 block along the reduction
 * dimension, as for the forward activations, is the project's reading. */
void oracle_gemm_1x128(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                       int64_t M, int64_t N, int64_t K, double *y)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < M * N; ++i)
        y[i] = gemm_element_g(xq, xs, wq, ws, K, i / N, i % N, i % N);
}

void oracle_gemm_1x128_sampled(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                               int64_t M, int64_t N, int64_t K, const int64_t *rows, const int64_t *cols,
                               int64_t count, double *y)
{
    int64_t i;
    (void)M;
    (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i)
        y[i] = gemm_element_g(xq, xs, wq, ws, K, rows[i], cols[i], cols[i]);
}

/* Grouped (MoE) GEMM: rows offs[e] .. offs[e+1]-1 of (xq, xs) use expert e's
 * weights wq[e] [N, K] and scales ws[e] [N/128, K/128]; rows never mix experts.
 * READING: the caller groups the rows by expert; empty groups are legal. */
static int64_t expert_of_row(const int32_t *offs, int64_t E, int64_t r)
{
    int64_t e;
    for (e = 0; e < E; ++e)
        if (r >= offs[e] && r < offs[e + 1])
            return e;
    return -1;
}

void oracle_grouped_gemm_sampled(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                                 const int32_t *offs, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                 const int64_t *rows, const int64_t *cols, int64_t count, double *y)
{
    int64_t i, wstride = N * K, sstride = (N / 128) * (K / 128);
    (void)M_total;
#pragma omp parallel for schedule(dynamic, 16)
    for (i = 0; i < count; ++i) {
        int64_t e = expert_of_row(offs, E, rows[i]);
        y[i] = (e < 0) ? NAN : gemm_element(xq, xs, wq + e * wstride, ws + e * sstride, K, rows[i], cols[i]);
    }
}

void oracle_grouped_gemm(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                         const int32_t *offs, int64_t E, int64_t M_total, int64_t N, int64_t K, double *y)
{
    int64_t i, wstride = N * K, sstride = (N / 128) * (K / 128);
#pragma omp parallel for schedule(static)
    for (i = 0; i < M_total * N; ++i) {
        int64_t r = i / N, e = expert_of_row(offs, E, r);
        y[i] = (e < 0) ? NAN : gemm_element(xq, xs, wq + e * wstride, ws + e * sstride, K, r, i % N);
    }
}

/* ---- the same GEMMs, every output, at full configuration sizes ------------
 *
 * gemm_element re-decodes both codes of every product.  The functions below
 * compute exactly the same numbers with the codes decoded once:
 *   - a 256-entry table holds decode(c) * 2^9 for every code c, filled from
 *     oracle_e4m3_decode (NaN for the two NaN codes);
 *   - X and W are turned into fp64 arrays of those integers;
 *   - each 128-wide block's dot product is summed in fp64.  Every product is an
 *     integer below 2^36 in magnitude (229376^2 < 2^36) and every partial sum
 *     of at most 128 of them an integer below 2^43 < 2^53, so each addition is
 *     exact whatever the order: the block sum equals gemm_element's int64 P.
 *     (That is why the compiler may vectorize the reduction.)
 *   - the scale product, the 2^-18 and the sum over blocks in ascending kb are
 *     the same fp64 operations as in gemm_element, so every output is
 *     bit-identical to oracle_gemm's.  A NaN code makes its outputs NaN.
 * Outputs are computed in tiles of TR rows x TC columns so that a tile's
 * operands stay in cache; the arithmetic per output is unchanged. */

static double e4m3_x512_table[256];

static void build_e4m3_x512_table(void)
{
    int c;
    for (c = 0; c < 256; ++c)
        e4m3_x512_table[c] = ldexp(oracle_e4m3_decode((uint32_t)c), 9);
}

/* the table, for the tests that pin it against oracle_e4m3_decode */
void oracle_e4m3_x512_table(double *out)
{
    int c;
    build_e4m3_x512_table();
    for (c = 0; c < 256; ++c)
        out[c] = e4m3_x512_table[c];
}

static void decode_x512(const uint8_t *q, int64_t n, double *d)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        d[i] = e4m3_x512_table[q[i]];
}

static double block_dot(const double *a, const double *b)
{
    double p = 0.0;
    int k;
#pragma omp simd reduction(+ : p)
    for (k = 0; k < 128; ++k)
        p += a[k] * b[k];
    return p;
}

enum { TR = 8, TC = 32 };

/* Rows r0 .. r1-1 of Y = X W^T from decoded operands; ws_of_col selects the
 * weight-scale layout: 0 = [N/128, K/128] blocks, 1 = [N, K/128] rows. */
static void gemm_rows_decoded(const double *xd, const float *xs, const double *wd, const float *ws, int64_t r0,
                              int64_t r1, int64_t N, int64_t K, int ws_of_col, double *y)
{
    int64_t KB = K / 128, tiles_r = (r1 - r0 + TR - 1) / TR, tiles_c = (N + TC - 1) / TC, t;
#pragma omp parallel for schedule(dynamic, 4)
    for (t = 0; t < tiles_r * tiles_c; ++t) {
        int64_t m0 = r0 + (t / tiles_c) * TR, n0 = (t % tiles_c) * TC, m, n, kb;
        int64_t m1 = m0 + TR < r1 ? m0 + TR : r1, n1 = n0 + TC < N ? n0 + TC : N;
        for (m = m0; m < m1; ++m)
            for (n = n0; n < n1; ++n)
                y[m * N + n] = 0.0;
        for (kb = 0; kb < KB; ++kb)
            for (m = m0; m < m1; ++m)
                for (n = n0; n < n1; ++n) {
                    double p = block_dot(xd + m * K + kb * 128, wd + n * K + kb * 128);
                    int64_t wrow = ws_of_col ? n : n / 128;
                    y[m * N + n] += ((double)xs[m * KB + kb] * (double)ws[wrow * KB + kb]) * ldexp(p, -18);
                }
    }
}

/* Work arrays for the decoded operands; 0 on success, -1 if out of memory. */
static int gemm_full(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M, int64_t N,
                     int64_t K, int ws_of_col, double *y)
{
    double *xd = (double *)malloc((size_t)(M * K > 0 ? M * K : 1) * sizeof(double));
    double *wd = (double *)malloc((size_t)(N * K > 0 ? N * K : 1) * sizeof(double));
    if (!xd || !wd) {
        free(xd);
        free(wd);
        return -1;
    }
    build_e4m3_x512_table();
    decode_x512(xq, M * K, xd);
    decode_x512(wq, N * K, wd);
    gemm_rows_decoded(xd, xs, wd, ws, 0, M, N, K, ws_of_col, y);
    free(xd);
    free(wd);
    return 0;
}

/* oracle_gemm, every output, bit-identical. */
int oracle_gemm_full(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M, int64_t N,
                     int64_t K, double *y)
{
    return gemm_full(xq, xs, wq, ws, M, N, K, 0, y);
}

/* oracle_gemm_1x128, every output, bit-identical. */
int oracle_gemm_1x128_full(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws, int64_t M,
                           int64_t N, int64_t K, double *y)
{
    return gemm_full(xq, xs, wq, ws, M, N, K, 1, y);
}

/* oracle_grouped_gemm, every output, bit-identical: each run of consecutive
 * rows that expert_of_row gives the same expert e is multiplied by expert e's
 * weights; rows no expert contains are NaN. */
int oracle_grouped_gemm_full(const uint8_t *xq, const float *xs, const uint8_t *wq, const float *ws,
                             const int32_t *offs, int64_t E, int64_t M_total, int64_t N, int64_t K, double *y)
{
    int64_t wstride = N * K, sstride = (N / 128) * (K / 128), b, t, n, decoded = -1;
    double *xd = (double *)malloc((size_t)(M_total * K > 0 ? M_total * K : 1) * sizeof(double));
    double *wd = (double *)malloc((size_t)(wstride > 0 ? wstride : 1) * sizeof(double));
    if (!xd || !wd) {
        free(xd);
        free(wd);
        return -1;
    }
    build_e4m3_x512_table();
    decode_x512(xq, M_total * K, xd);
    for (b = 0; b < M_total; b = t) {
        int64_t e = expert_of_row(offs, E, b);
        for (t = b + 1; t < M_total && expert_of_row(offs, E, t) == e; ++t)
            ;
        if (e < 0) {
            for (n = b * N; n < t * N; ++n)
                y[n] = NAN;
            continue;
        }
        if (e != decoded) {
            decode_x512(wq + e * wstride, wstride, wd);
            decoded = e;
        }
        gemm_rows_decoded(xd, xs, wd, ws + e * sstride, b, t, N, K, 0, y);
    }
    free(xd);
    free(wd);
    return 0;
}

/* ---- attention over an FP8 KV cache ---------------------------------------
 *
 * The article's section "Real-world performance gains" reports that keeping
 * the KV cache and attention in FP8 as well raises the end-to-end gain from
 * the linear layers' 15-25% to about 48%.  It gives no granularity.
 * READING: the cache stores keys and values as E4M3 codes with one fp32 scale
 * per (token, head) -- a 1x128 block along the head dimension D = 128, i.e.
 * quant_act_1x128 of the [tokens, heads * 128] key and value rows -- and the
 * attention of a new query token reads the dequantized cache:
 *   s_j = sm_scale * sum_d q[d] * (decode(kq[j, d]) * ks[j]),   j < len,
 *   p_j = exp(s_j - max_i s_i) / sum_i exp(s_i - max_i s_i),
 *   o[d] = sum_j p_j * (decode(vq[j, d]) * vs[j]).
 * Query head h reads key/value head h / (Hq / Hkv) (grouped queries).  The
 * query is bf16.  An empty context (len = 0) gives o = 0 (READING).
 * Everything is fp64 here; layouts:
 *   q [B, Hq, 128] bf16; kq, vq [B, T, Hkv, 128] codes; ks, vs [B, T, Hkv];
 *   lens [B] (entries clamped to [0, T]); out [B, Hq, 128] fp64. */
void oracle_kv_attention_decode(const uint16_t *q, const uint8_t *kq, const float *ks, const uint8_t *vq,
                                const float *vs, const int32_t *lens, int64_t B, int64_t T, int64_t Hq,
                                int64_t Hkv, double sm_scale, double *out)
{
    const int64_t D = 128;
    int64_t bh;
#pragma omp parallel for schedule(dynamic, 1)
    for (bh = 0; bh < B * Hq; ++bh) {
        int64_t b = bh / Hq, h = bh % Hq, g = h / (Hq / Hkv), j, d;
        int64_t len = lens[b] < 0 ? 0 : (lens[b] > T ? T : lens[b]);
        double *o = out + bh * D, smax = -INFINITY, denom = 0.0;
        double *sc = (double *)malloc((size_t)(len > 0 ? len : 1) * sizeof(double));
        for (d = 0; d < D; ++d)
            o[d] = 0.0;
        for (j = 0; j < len; ++j) {
            const int64_t kv = (b * T + j) * Hkv + g;
            double dot = 0.0;
            for (d = 0; d < D; ++d)
                dot += (double)bf16_value(q[bh * D + d]) * (oracle_e4m3_decode(kq[kv * D + d]) * (double)ks[kv]);
            sc[j] = sm_scale * dot;
            if (sc[j] > smax)
                smax = sc[j];
        }
        for (j = 0; j < len; ++j) {
            const int64_t kv = (b * T + j) * Hkv + g;
            const double p = exp(sc[j] - smax);
            denom += p;
            for (d = 0; d < D; ++d)
                o[d] += p * (oracle_e4m3_decode(vq[kv * D + d]) * (double)vs[kv]);
        }
        if (len > 0)
            for (d = 0; d < D; ++d)
                o[d] /= denom;
        free(sc);
    }
}

/* ---- threading ------------------------------------------------------------- */

int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
