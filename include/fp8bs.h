/*
 * fp8bs.h -- C ABI of the block-scaled FP8 linear-layer library for AMD
 * Instinct MI355X (gfx950, CDNA4).
 *
 * The method: the article "NVIDIA NeMo RL achieves 48% speedup with end-to-end
 * FP8 precision training" (Jessie A Ellis, Apr 20 2026; mexc.co/hi-IN/news/
 * 1041474 and its two translations).  Its section "Technical breakthrough"
 * quantizes block-wise to FP8 E4M3 -- one block of 128x128 for weights, 1x128
 * for activations -- and runs the linear layers in FP8 math.  Its section
 * "Real-world performance gains" recalibrates the quantization scales after
 * every training step and reports a matching accuracy on a mixture-of-experts
 * model.  Its closing section offers power-of-2 scaling factors.  The article
 * prints no formula: the scale rule (amax / 448), the rounding (saturating
 * round-to-nearest-even of the correctly rounded fp32 quotient), fp32 scales
 * applied per 128-wide K block, and the grouped MoE form are this library's
 * statement of the method.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is a DEVICE pointer owned by the caller; the library
 *   allocates nothing.  Tensors are dense and row-major.
 * - bf16 tensors are passed as raw 16-bit payloads.  FP8 codes are bytes in
 *   the OCP E4M3FN encoding (bias 7, largest finite 448, NaN = S.1111.111).
 * - Scales are fp32 DEQUANTIZATION multipliers: x ~= decode(q) * s.
 * - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is the
 *   null stream).  The library never synchronizes; results are ready when the
 *   stream reaches them.  Calls are reentrant; repeated calls with the same
 *   arguments produce bit-identical results (no atomics in any reduction).
 * - Return value: FP8BS_OK (0) or one of the status codes below.  Arguments
 *   are checked before any device work is enqueued, so a non-zero return
 *   means nothing was launched, except FP8BS_HIP_ERROR, which reports a
 *   failed launch.  No C++ exception and no abort crosses this boundary.
 * - M == 0 (or M_total == 0) is a valid no-op.  K and N must be multiples of
 *   128.  Tensor pointers must be 16-byte aligned, scale pointers 4-byte
 *   aligned.  Non-finite inputs are outside the contract: the output is then
 *   unspecified, but no kernel reads or writes out of bounds.
 */
#ifndef FP8BS_H
#define FP8BS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8BS_ABI_VERSION 2

/* Symbols of this header are the only ones the shared library exports. */
#if defined(__GNUC__) || defined(__clang__)
#define FP8BS_API __attribute__((visibility("default")))
#else
#define FP8BS_API
#endif

enum fp8bs_status {
    FP8BS_OK = 0,
    FP8BS_INVALID_ARG = 1,         /* null pointer with a non-zero extent, negative size, misaligned
                                      pointer, unknown enum value */
    FP8BS_UNSUPPORTED_SHAPE = 2,   /* K (or N where required) not a multiple of 128; size too large */
    FP8BS_UNSUPPORTED_DEVICE = 3,  /* the current HIP device is not a gfx950 */
    FP8BS_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes below the size the query function returns */
    FP8BS_HIP_ERROR = 5,           /* the HIP runtime refused a launch */
    FP8BS_SCRATCH_TOO_SMALL = 6    /* fp8_block_grouped_gemm_noalloc: the problem's row-tile tables
                                      exceed FP8BS_NOALLOC_SCRATCH_BYTES */
};

/* scale_mode */
enum fp8bs_scale_mode {
    FP8BS_SCALE_EXACT = 0, /* s = RN_fp32(amax / 448); the largest element maps to +-448 */
    FP8BS_SCALE_POW2 = 1   /* s = 2^k, the least k with amax <= 448 * 2^k (never clips) */
};

/* out_dtype */
enum fp8bs_out_dtype {
    FP8BS_OUT_BF16 = 0, /* bf16 payloads, round-to-nearest-even of the fp32 result */
    FP8BS_OUT_FP32 = 1  /* the fp32 accumulator itself */
};

/*
 * quant_act_1x128 -- activation quantizer, one scale per 1x128 row block
 * (article section "Technical breakthrough": 1x128 granularity for
 * activations).
 *
 *   x_bf16 : [M, K] bf16 payloads (input, read only)
 *   xq     : [M, K] E4M3 codes (output)
 *   xs     : [M, K/128] fp32 scales (output); xs[m, kb] covers
 *            x[m, 128*kb .. 128*kb+127]
 *
 * For each block: amax = max |x| (exact); s = scale(amax, scale_mode), with
 * s = 1 for an all-zero block; q = E4M3_sat_RNE(RN_fp32(x / s)), the sign of
 * x (also of -0) kept in the code.  Bit-exact and deterministic.
 * Errors: INVALID_ARG (null x/xq/xs with M > 0, M < 0, K <= 0, misalignment,
 * bad scale_mode), UNSUPPORTED_SHAPE (K % 128 != 0), UNSUPPORTED_DEVICE.
 */
FP8BS_API int quant_act_1x128(const void *x_bf16, int64_t M, int64_t K, void *xq, float *xs, int scale_mode,
                    void *stream);

/*
 * quant_act_1x128_t -- quant_act_1x128 of the transpose: X [M, K] quantized
 * in 1x128 blocks that run down its columns (128 consecutive rows of one
 * column), written transposed.  The weight gradient dW = dY^T X of a
 * training step contracts over the tokens, so both of its operands are
 * quantized along them (the article's recipe runs FP8 in training as well,
 * section "Technical breakthrough"; the block runs along the reduction
 * dimension, as the 1x128 activation block does in the forward product).
 *
 *   x_bf16 : [M, K] bf16 payloads (input), M and K multiples of 128
 *   xqt    : [K, M] E4M3 codes, row k = the codes of column k of X
 *   xst    : [K, M/128] fp32 scales; xst[k, mb] covers X[128 mb .. 128 mb + 127, k]
 * Bit for bit quant_act_1x128 of the transposed matrix (the same element
 * rule, amax over a block's 128 values).  Errors: as quant_act_1x128, and
 * UNSUPPORTED_SHAPE if M % 128 != 0.  M == 0 is a no-op.
 */
FP8BS_API int quant_act_1x128_t(const void *x_bf16, int64_t M, int64_t K, void *xqt, float *xst, int scale_mode,
                                void *stream);

/*
 * quant_act_1x128_dual -- quant_act_1x128 and quant_act_1x128_t of the same
 * X [M, K] from one read of X: (xq [M, K], xs [M, K/128]) exactly as
 * quant_act_1x128 writes them, and (xqt [K, M], xst [K, M/128]) exactly as
 * quant_act_1x128_t does.  A training step quantizes each output gradient
 * dY both ways: along its rows for the data gradient dX = dY W, along the
 * tokens for the weight gradient dW = dY^T X.  Errors: as quant_act_1x128_t,
 * and INVALID_ARG for a null or misaligned output.  M == 0 is a no-op.
 */
FP8BS_API int quant_act_1x128_dual(const void *x_bf16, int64_t M, int64_t K, void *xq, float *xs, void *xqt,
                                   float *xst, int scale_mode, void *stream);

/*
 * quant_act_1x128_gather -- the activation quantizer over gathered rows: the
 * MoE dispatch.  The article runs its recipe on a mixture-of-experts model
 * (section "Real-world performance gains"); an MoE layer's grouped GEMM takes
 * each token's row once per expert it is routed to, in expert order.  The
 * 1x128 blocks lie along a row, so this equals quant_act_1x128 of the
 * gathered matrix, computed without materializing it.
 *
 *   x_bf16 : [T, K] bf16 payloads (input): the token rows
 *   rows   : [M] int32 row indices into x (device memory, never read by the
 *            host)
 *   xq     : [M, K] E4M3 codes (output); xs : [M, K/128] fp32 scales (output)
 *
 * xq[m], xs[m] = quant_act_1x128(x[rows[m]]), bit for bit.  An index outside
 * [0, T) yields an all-zero row (codes 0, scales 1); no memory outside x is
 * read.  Errors: INVALID_ARG (T < 0, M < 0, K <= 0, bad scale_mode, null or
 * misaligned x (16 B, when T > 0), rows (4 B), xq (16 B), xs (4 B) with
 * M > 0), UNSUPPORTED_SHAPE (K % 128 != 0, M * K / 128 >= 2^31),
 * UNSUPPORTED_DEVICE.  M == 0 is a no-op.
 */
FP8BS_API int quant_act_1x128_gather(const void *x_bf16, int64_t T, int64_t K, const int32_t *rows, int64_t M,
                                     void *xq, float *xs, int scale_mode, void *stream);

/*
 * quant_act_1x128_scatter -- the MoE dispatch from the token side: each token
 * row is read and quantized once, and its codes and scales are written to
 * every row the routing sends it to (the same result as quant_act_1x128_gather
 * with the inverse map, with each token row read once instead of once per
 * expert).
 *
 *   x_bf16 : [T, K] bf16 payloads (input): the token rows
 *   dest   : [T, topk] int32 destination rows (device memory, never read by
 *            the host): token t goes to rows dest[t * topk + k], k < topk
 *   xq     : [M, K] E4M3 codes (output); xs : [M, K/128] fp32 scales (output)
 *
 * For every entry d = dest[t * topk + k] with 0 <= d < M: xq[d], xs[d] =
 * quant_act_1x128(x[t]), bit for bit.  Entries outside [0, M) are skipped;
 * rows that no entry names are not written.  Two entries naming the same row
 * leave one of the two token rows there (which one is unspecified).  Errors:
 * INVALID_ARG (negative sizes, bad scale_mode, null or misaligned x (16 B),
 * dest (4 B), xq (16 B), xs (4 B) when T, topk and M are all positive),
 * UNSUPPORTED_SHAPE (K % 128 != 0, a size or block count >= 2^31),
 * UNSUPPORTED_DEVICE.  T, topk or M == 0 is a no-op.
 */
FP8BS_API int quant_act_1x128_scatter(const void *x_bf16, int64_t T, int64_t K, const int32_t *dest, int64_t topk,
                                      int64_t M, void *xq, float *xs, int scale_mode, void *stream);

/*
 * swiglu_quant_1x128 -- the MLP's gated activation fused with the 1x128
 * activation quantizer of the down projection's input.  The article keeps
 * non-linear functions in BF16 and runs the linear layers in FP8 (section
 * "Technical breakthrough"), and counts quantization kernel overhead in the
 * gap to the 2x peak (section "Real-world performance gains"); this entry
 * point takes the gate+up projection's output to the down projection's FP8
 * input in one pass.
 *
 *   gu_bf16 : [M, 2F] bf16 payloads (input): columns 0..F-1 of a row are the
 *             gate values g, columns F..2F-1 the up values u
 *   hq      : [M, F] E4M3 codes (output)
 *   hs      : [M, F/128] fp32 scales (output)
 *
 * h[m, f] = the bf16 value nearest (ties to even) to (g * sigma(g)) * u
 * evaluated in fp64 with sigma(g) = 1 / (1 + exp(-g)), g = gu[m, f],
 * u = gu[m, F + f]; then (hq, hs) = quant_act_1x128(h, scale_mode), bit for
 * bit.  (The fp64 evaluation decides only where h lies within about 2^-50 of
 * a bf16 rounding midpoint.)  Results are unspecified where |g * u| exceeds
 * the bf16 range or an input is not finite.
 * Errors: INVALID_ARG (null or misaligned gu_bf16/hq (16 B) or hs (4 B) with
 * M > 0, M < 0, F <= 0, bad scale_mode), UNSUPPORTED_SHAPE (F % 128 != 0, or
 * M * F / 128 >= 2^31), UNSUPPORTED_DEVICE.  M == 0 is a no-op.
 */
FP8BS_API int swiglu_quant_1x128(const void *gu_bf16, int64_t M, int64_t F, void *hq, float *hs, int scale_mode,
                                 void *stream);

/*
 * quant_w_128x128 -- weight quantizer, one scale per 128x128 block (article
 * section "Technical breakthrough": 128x128 granularity for weights).  Called
 * on every weight after each optimizer step, it is the per-step scale
 * recalibration of section "Real-world performance gains".
 *
 *   w_bf16 : [N, K] bf16 payloads (input)
 *   wq     : [N, K] E4M3 codes (output)
 *   ws     : [N/128, K/128] fp32 scales (output); ws[nb, kb] covers rows
 *            128*nb .. 128*nb+127, columns 128*kb .. 128*kb+127
 *
 * Same element rule as quant_act_1x128, with amax over the 16384 values of a
 * block.  Errors: as quant_act_1x128, and UNSUPPORTED_SHAPE if N % 128 != 0.
 */
FP8BS_API int quant_w_128x128(const void *w_bf16, int64_t N, int64_t K, void *wq, float *ws, int scale_mode,
                    void *stream);

/*
 * quant_w_128x128_batched -- the weight quantizer over `count` independent
 * tensors in one launch (the recalibration of every weight of a model after
 * a step).  w_bf16[i], wq[i], ws[i], N[i], K[i] describe tensor i exactly as
 * in quant_w_128x128.  The five arrays are HOST arrays of `count` entries,
 * read during the call only; the pointers they hold are device pointers.
 * Errors: as quant_w_128x128 for any tensor; INVALID_ARG if count < 0 or an
 * array is null with count > 0.  count == 0 is a no-op.
 */
FP8BS_API int quant_w_128x128_batched(int64_t count, const void *const *w_bf16, const int64_t *N,
                            const int64_t *K, void *const *wq, float *const *ws, int scale_mode,
                            void *stream);

/*
 * quant_w_128x128_dual -- the weight quantizer for training: the codes and
 * scales of W and, from the same read of W, those of its transpose.  The
 * article's recipe runs FP8 in training as well as in generation (section
 * "Technical breakthrough"); the backward product dX = dY W multiplies by
 * W^T, whose 128x128 blocks are W's blocks transposed, so block (kb, nb) of
 * W^T has the amax, scale and codes of block (nb, kb) of W, moved.
 *
 *   w_bf16 : [N, K] bf16 payloads (input)
 *   wq, ws : exactly as quant_w_128x128 writes them ([N, K], [N/128, K/128])
 *   wqt    : [K, N] E4M3 codes, wqt[k, n] = wq[n, k]
 *   wst    : [K/128, N/128] fp32 scales, wst[kb, nb] = ws[nb, kb]
 * so (wqt, wst) equals quant_w_128x128 of the transposed matrix, and
 * fp8_block_gemm(dyq, dys, wqt, wst, M, K, N) is the data gradient for
 * dY [M, N] quantized by quant_act_1x128.  All outputs are caller-owned
 * device buffers; wqt and wq are 16-byte aligned, the scales 4-byte aligned.
 * Errors: as quant_w_128x128, and INVALID_ARG for a null or misaligned
 * transposed output.
 */
FP8BS_API int quant_w_128x128_dual(const void *w_bf16, int64_t N, int64_t K, void *wq, float *ws, void *wqt,
                                   float *wst, int scale_mode, void *stream);

/*
 * quant_w_128x128_dual_batched -- quant_w_128x128_dual over `count` tensors
 * in one launch (per-step recalibration of a model's weights for training).
 * The seven arrays are HOST arrays of `count` entries, read during the call
 * only; the pointers they hold are device pointers.  Errors: as
 * quant_w_128x128_dual for any tensor; INVALID_ARG if count < 0 or an array
 * is null with count > 0.  count == 0 is a no-op.
 */
FP8BS_API int quant_w_128x128_dual_batched(int64_t count, const void *const *w_bf16, const int64_t *N,
                                           const int64_t *K, void *const *wq, float *const *ws,
                                           void *const *wqt, float *const *wst, int scale_mode, void *stream);

/*
 * fp8_block_gemm -- Y = dequant(Xq) * dequant(Wq)^T, the FP8 linear layer
 * (article section "Technical breakthrough": linear layers run FP8 math).
 *
 *   xq [M, K] E4M3, xs [M, K/128] fp32     (from quant_act_1x128)
 *   wq [N, K] E4M3, ws [N/128, K/128] fp32 (from quant_w_128x128)
 *   y  [M, N] bf16 payloads or fp32 (out_dtype)
 *
 *   Y[m, n] = sum_kb (xs[m, kb] * ws[n/128, kb]) * P[m, n, kb],
 *   P[m, n, kb] = sum_{k in block kb} decode(xq[m, k]) * decode(wq[n, k]),
 * where P comes from FP8 matrix-core products accumulated in fp32 and the
 * scale product is formed and applied in fp32 per 128-wide K block (for a
 * single row, M == 1 with K <= 16384, the products and sums run on the
 * vector ALUs in fp32 instead).  The order of the additions is the
 * hardware's, and the matrix cores sum a K block's 128 products at reduced
 * precision when one product dominates (below 2^-12 of the block's sum of
 * |products| in every measured case), so results agree with an exact
 * evaluation closely, not bit for bit; the bf16 output is the
 * round-to-nearest-even of exactly the value the fp32 output holds.
 * A given (M, N, K) always runs the same kernel: results are deterministic.
 *
 *   workspace, workspace_bytes: device scratch for the fp32 partial sums of
 *   products split along K (shapes with fewer 256-wide output tiles than the
 *   GPU has compute units, e.g. decode-sized M): ksplit * M * N * 4 bytes,
 *   as fp8bs_gemm_workspace_size(M, N, K) returns (0 for the other shapes,
 *   where workspace may be NULL).  It need not be zeroed; its contents are
 *   overwritten.  Two calls that share a workspace must not overlap in time.
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE (N or K not a multiple of 128, or
 *   ceil(M / 128) * N / 128 of 2^31 or more output tiles),
 * WORKSPACE_TOO_SMALL, UNSUPPORTED_DEVICE, HIP_ERROR.
 */
FP8BS_API int fp8_block_gemm(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                   int64_t K, void *y, int out_dtype, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * fp8_block_gemm_1x128 -- fp8_block_gemm with 1x128 scales on both operands:
 *   Y[m, n] = sum_kb (xs[m, kb] * ws[n, kb]) * P[m, n, kb],
 * ws [N, K/128] holding one scale per row of wq and K block.  This is the
 * weight gradient of a training step, dW = dY^T X, with
 *   xq, xs = quant_act_1x128_t(dY)  ([N_out, M_tok], rows of dY^T),
 *   wq, ws = quant_act_1x128_t(X)   ([K_in, M_tok], rows of X^T),
 * so M = N_out, N = K_in, K = M_tok and Y [N_out, K_in] is dW.  The scale
 * product is formed in fp32 per output element and K block, then applied by
 * one fp32 FMA into the accumulator.  The bf16 output is the round to
 * nearest even of the fp32 output.  Errors: INVALID_ARG, UNSUPPORTED_SHAPE
 * (N or K not a multiple of 128), UNSUPPORTED_DEVICE, HIP_ERROR.  No
 * workspace.  M == 0 is a no-op.
 */
FP8BS_API int fp8_block_gemm_1x128(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M,
                                   int64_t N, int64_t K, void *y, int out_dtype, void *stream);

/*
 * fp8_block_gemm_1x128_pow2 -- fp8_block_gemm_1x128 for operands quantized
 * with power-of-2 scales (the article's closing section; scale_mode
 * FP8BS_SCALE_POW2 of quant_act_1x128_t).  Arguments, layouts and errors are
 * those of fp8_block_gemm_1x128, with the precondition of fp8_block_gemm_pow2
 * on every xs and ws entry.  On the large-tile kernels both per-row scales go
 * to the matrix cores' E8M0 operands (each lane passes the scale of the row of
 * xq and of wq that it holds), so the MFMA accumulates 2^(ex + ew) * P
 * directly, with no fp32 rescale pass; the results agree with
 * fp8_block_gemm_1x128 on the same operands to within fp32 rounding of the
 * accumulation order.
 */
FP8BS_API int fp8_block_gemm_1x128_pow2(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M,
                                        int64_t N, int64_t K, void *y, int out_dtype, void *stream);

/*
 * fp8_block_grouped_gemm -- the MoE (mixture-of-experts) form of
 * fp8_block_gemm (article section "Real-world performance gains": the recipe
 * on Qwen3-30B, a mixture-of-experts model).
 *
 *   xq [M_total, K], xs [M_total, K/128]: token rows grouped by expert
 *   wq [E, N, K], ws [E, N/128, K/128]: one weight matrix per expert
 *   group_offsets: DEVICE int32 [E + 1]; rows group_offsets[e] ..
 *     group_offsets[e+1]-1 belong to expert e.  The caller guarantees
 *     group_offsets[0] == 0, non-decreasing, group_offsets[E] == M_total.
 *     The host never reads them.  Empty groups are legal.  Offsets outside
 *     [0, M_total] are clamped by the kernel, so they cannot cause an
 *     out-of-bounds access (the result is then unspecified).
 *   y [M_total, N]: row r holds fp8_block_gemm of row r with its expert.
 * Workspace: fp8bs_grouped_workspace_size(E, M_total, N, K) bytes: 16 for
 *   the row-tile counts, then 16 per row tile: at most ceil(M_total / 256) + E
 *   tiles of 256 rows and E short last tiles (an expert's last <= 128 rows,
 *   multiplied with 128-row tiles instead of padded to 256).  The call first
 *   writes the counts and the tables of (expert, first row, row count) there
 *   from group_offsets, on the device.  It need not be zeroed; calls that
 *   share a workspace must not overlap in time.
 * Errors: as fp8_block_gemm; INVALID_ARG if E <= 0 with M_total > 0.
 */
FP8BS_API int fp8_block_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                           const int32_t *group_offsets, int64_t E, int64_t M_total, int64_t N, int64_t K,
                           void *y, int out_dtype, void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp8_block_gemm_pow2, fp8_block_grouped_gemm_pow2 -- the two GEMMs for
 * operands quantized with power-of-2 scales (the power-of-2 scaling option in
 * the article's closing section; scale_mode FP8BS_SCALE_POW2 of the
 * quantizers).  Arguments, layouts, workspace and errors are exactly those of
 * fp8_block_gemm and fp8_block_grouped_gemm.
 *
 * Precondition: every xs and ws entry is a power of two no smaller than
 * 2^-127 (the E8M0 range; POW2 quantization gives that for every block whose
 * amax is at least 448 * 2^-127, about 2.6e-36).  On the large-tile kernels
 * each K block's two scales go to the matrix cores' E8M0 block-scale
 * operands, the weight scale on the weight operand and the activation row's
 * scale on the activation operand, so the MFMA accumulates
 * 2^(ex + ew) * P directly, exactly, with no fp32 rescale pass, even where
 * the product of the two scales lies below fp32's normal range.  Only each
 * scale's exponent is used there; with scales that break the precondition
 * the result is unspecified (it is never a memory fault).  Results agree with
 * fp8_block_gemm on the same operands to within fp32 rounding of the
 * accumulation order; the bf16 output is again the round-to-nearest-even of
 * the fp32 output of the same call shape.
 */
FP8BS_API int fp8_block_gemm_pow2(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M,
                                  int64_t N, int64_t K, void *y, int out_dtype, void *workspace,
                                  size_t workspace_bytes, void *stream);
FP8BS_API int fp8_block_grouped_gemm_pow2(const void *xq, const float *xs, const void *wq, const float *ws,
                                          const int32_t *group_offsets, int64_t E, int64_t M_total, int64_t N,
                                          int64_t K, void *y, int out_dtype, void *workspace,
                                          size_t workspace_bytes, void *stream);

/*
 * fp8_block_gemm_quant -- the block-scaled GEMM whose output is also the next
 * FP8 layer's input: Y = fp8_block_gemm(xq, xs, wq, ws) in bf16, together with
 * quant_act_1x128(Y), computed in the GEMM's epilogue where the shape allows
 * (article section "Real-world performance gains": quantization kernels are
 * one of the two costs that keep the linear-layer gain below the FP8 peak's
 * 2x; quantizing in the producing kernel removes the separate pass over Y).
 *   xq, xs, wq, ws, M, N, K: as fp8_block_gemm (K and N multiples of 128).
 *   scale_mode: FP8BS_SCALE_EXACT or FP8BS_SCALE_POW2 -- the scales of the
 *     operands (POW2: as fp8_block_gemm_pow2, with its precondition) and of
 *     the output's quantization.
 *   y: bf16 [M, N] (round to nearest even of the fp32 accumulator), or NULL
 *     when only the quantized output is wanted.
 *   yq [M, N] codes and ys [M, N/128] fp32 scales: bit for bit what
 *     quant_act_1x128(Y, scale_mode) writes for this call's bf16 Y.
 * Workspace: fp8bs_gemm_quant_workspace_size(M, N, K) bytes, 0 where the
 *   quantization runs in the GEMM's epilogue (the large products: each
 *   256 x 256 output tile's waves hold whole 128-column blocks of their rows);
 *   elsewhere a bf16 Y buffer (used when y is NULL) followed by
 *   fp8_block_gemm's own workspace, and the quantizer runs as a second launch.
 * Errors: as fp8_block_gemm; y may be NULL, yq and ys may not (unless M == 0).
 */
FP8BS_API size_t fp8bs_gemm_quant_workspace_size(int64_t M, int64_t N, int64_t K);
FP8BS_API int fp8_block_gemm_quant(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M,
                                   int64_t N, int64_t K, void *y, void *yq, float *ys, int scale_mode,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * fp8_kv_attention_decode -- attention of one new query token per sequence
 * over an FP8 KV cache (rollout decode; article section "Real-world
 * performance gains": an FP8 KV cache and FP8 attention lift the end-to-end
 * gain to about 48%).
 *   q [B, Hq, 128] bf16: the query heads of each sequence's new token.
 *   kq, vq [B, T, Hkv, 128] E4M3 codes and ks, vs [B, T, Hkv] fp32 scales:
 *     keys and values cached with one scale per (token, head) -- exactly
 *     quant_act_1x128 of the [B * T, Hkv * 128] key and value rows, so a
 *     cache is filled (or a token appended at row b * T + t) by that call.
 *   lens: DEVICE int32 [B]; sequence b attends to its cached tokens
 *     0 .. lens[b] - 1 (clamped to [0, T]; an empty context gives 0).
 *   Query head h reads key/value head h / (Hq / Hkv); Hq / Hkv must be 1, 2,
 *     4 or 8 (grouped queries).  The head dimension is 128.
 *   o[b, h, :] = sum_j softmax_j(sm_scale * ks * q . decode(k_j)) * vs * decode(v_j),
 *     written to out [B, Hq, 128] as bf16 (round to nearest even of the fp32
 *     result) or fp32 (out_dtype).  Scores use the matrix cores on bf16 (key
 *     codes decode exactly; products are exact), the rest is fp32.
 * Workspace: fp8bs_kv_attention_workspace_size(B, T, Hq, Hkv) bytes (the
 *   per-split partial states when a sequence's tokens are split over several
 *   workgroups; 0 otherwise).  It need not be zeroed.
 * Errors: INVALID_ARG for null/misaligned pointers, negative sizes, a
 *   non-finite sm_scale or an unknown out_dtype; UNSUPPORTED_SHAPE for other
 *   group sizes or T * Hkv * 128 >= 2^31; WORKSPACE_TOO_SMALL.
 */
FP8BS_API size_t fp8bs_kv_attention_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv);
FP8BS_API int fp8_kv_attention_decode(const void *q_bf16, const void *kq, const float *ks, const void *vq,
                                      const float *vs, const int32_t *lens, int64_t B, int64_t T, int64_t Hq,
                                      int64_t Hkv, float sm_scale, void *out, int out_dtype, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * fp8_block_grouped_gemm_noalloc -- fp8_block_grouped_gemm for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  It takes no workspace and calls no
 * hipMalloc, hipFree or other allocating routine.
 *
 * Arguments, layouts and results are those of fp8_block_grouped_gemm (EXACT
 * scales; the output is bit-identical to it).  The row-tile tables that
 * fp8_block_grouped_gemm writes into its workspace go instead to a static
 * device array of FP8BS_NOALLOC_SCRATCH_BYTES inside the library: one per
 * GPU, allocated when the library's code is loaded on that GPU and held until
 * the process ends.  Its address is looked up on the first call on each
 * device.  The tables are rewritten in full by every call, so nothing needs
 * clearing between calls.
 * Concurrency: every call on one GPU shares that GPU's array.  Calls that
 *   overlap in time on one GPU (different streams, or different host threads
 *   without ordering) race on it and give unspecified results; serialize them,
 *   e.g. on one stream.
 * Limit: the tables take 16 + 16 * (ceil(M_total / 256) + 2 E) bytes, i.e.
 *   fp8bs_grouped_workspace_size(E, M_total, N, K); about 65,500 row tiles fit
 *   (for instance M_total = 16M rows with E = 128).
 * Errors: as fp8_block_grouped_gemm, plus FP8BS_SCRATCH_TOO_SMALL (nothing
 *   launched) when the tables would exceed the array, and FP8BS_HIP_ERROR if
 *   the runtime cannot give the array's address.
 */
#define FP8BS_NOALLOC_SCRATCH_BYTES 1048576
FP8BS_API int fp8_block_grouped_gemm_noalloc(const void *xq, const float *xs, const void *wq, const float *ws,
                                             const int32_t *group_offsets, int64_t E, int64_t M_total, int64_t N,
                                             int64_t K, void *y, int out_dtype, void *stream);

/*
 * fp8_block_linear, fp8_block_linear_pow2 -- the whole FP8 linear layer from
 * bf16 activations: Y = fp8_block_gemm(quant_act_1x128(X), Wq, Ws) (article
 * section "Technical breakthrough": activations are quantized per 1x128
 * block as they enter each linear layer).  The _pow2 form quantizes X with
 * power-of-2 scales (FP8BS_SCALE_POW2) and runs fp8_block_gemm_pow2, whose
 * precondition ws must then meet.
 *
 *   x [M, K] bf16 payloads, row-major
 *   wq, ws, y, out_dtype: as fp8_block_gemm
 *
 * For one row (M == 1, K <= 16384) the vector-ALU product for single
 * activation rows quantizes x in registers; for at most 16 rows (decode) with
 * 8 <= K/128 <= 128 and N a multiple of 32 with N/32 >= 256, the
 * weight-streaming kernel does.  Either one uses the quantizer's own encoder,
 * so no quantized copy of x is written or read back.  Other shapes run
 * quant_act_1x128 into the workspace, then the GEMM.  Either way
 * y is bit for bit that of quant_act_1x128 followed by fp8_block_gemm (or the
 * _pow2 pair) on the same stream, with the default kernel selection (no
 * FP8BS_GEMM_VARIANT override).
 *
 * Workspace: fp8bs_linear_workspace_size(M, N, K) bytes (0 for the fused
 *   shapes, where workspace may be NULL): the quantized x, its scales, then
 *   the GEMM's own workspace, each 16-byte aligned.  (At M == 1 the size is
 *   still required, though the single-row product leaves it unused.)  It need not be zeroed;
 *   calls that share a workspace must not overlap in time.
 * Errors: as fp8_block_gemm (x takes xq's place), plus UNSUPPORTED_SHAPE for
 *   shapes quant_act_1x128 rejects.
 */
FP8BS_API int fp8_block_linear(const void *x_bf16, const void *wq, const float *ws, int64_t M, int64_t N, int64_t K,
                               void *y, int out_dtype, void *workspace, size_t workspace_bytes, void *stream);
FP8BS_API int fp8_block_linear_pow2(const void *x_bf16, const void *wq, const float *ws, int64_t M, int64_t N,
                                    int64_t K, void *y, int out_dtype, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Workspace size in bytes for fp8_block_linear(_pow2) of this shape (0 for
 * the fused decode shapes); no device call. */
FP8BS_API size_t fp8bs_linear_workspace_size(int64_t M, int64_t N, int64_t K);

/* Workspace sizes in bytes for the two GEMMs: functions of the shape (and of
 * the FP8BS_GEMM_VARIANT / FP8BS_GEMM_KSPLIT measurement overrides, read once
 * per process); no device call. */
FP8BS_API size_t fp8bs_gemm_workspace_size(int64_t M, int64_t N, int64_t K);
FP8BS_API size_t fp8bs_grouped_workspace_size(int64_t E, int64_t M_total, int64_t N, int64_t K);

/* Static, NUL-terminated description of a status code (never NULL). */
FP8BS_API const char *fp8bs_status_string(int status);

/* FP8BS_ABI_VERSION of the built library. */
FP8BS_API int fp8bs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8BS_H */
