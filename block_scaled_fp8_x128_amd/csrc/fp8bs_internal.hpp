// fp8bs_internal.hpp -- host-side launchers shared between the kernel files
// and the C ABI layer.  Every launcher enqueues on `stream` and returns the
// HIP status of the launch; argument checking happens in the ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <tuple>
#include <utility>

namespace fp8bs {

// Launch through hipLaunchKernel so that the status of THIS launch is
// returned (the <<<>>> form reports through hipGetLastError, which would also
// pick up an unrelated earlier error of the caller).
template <typename... KArgs, typename... Args>
static inline hipError_t launch(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem, hipStream_t stream,
                                Args... args)
{
    std::tuple<KArgs...> held(static_cast<KArgs>(args)...);
    void *ptrs[sizeof...(KArgs)];
    std::apply([&](auto &...a) {
        int i = 0;
        ((ptrs[i++] = (void *)&a), ...);
    }, held);
    return hipLaunchKernel((const void *)kern, grid, block, ptrs, shmem, stream);
}

// ---- quantizers (fp8bs_quant.hip) ------------------------------------------

hipError_t launch_quant_act(const void *x, int64_t M, int64_t K, void *xq, float *xs, int mode, hipStream_t stream);
// quant_act_1x128 of X^T: codes [K, M], scales [K, M/128] (M, K multiples of
// 128); with xq != nullptr also quant_act_1x128 of X itself (xq [M, K], xs
// [M, K/128]) from the same read.
hipError_t launch_quant_act_t(const void *x, int64_t M, int64_t K, void *xqt, float *xst, int mode,
                              hipStream_t stream, void *xq = nullptr, float *xs = nullptr);

// quant_act_1x128 of x[rows[m]] for m < M (x [T, K]; an index outside
// [0, T) reads as a zero row) (fp8bs_route.hip).
hipError_t launch_quant_act_gather(const void *x, int64_t T, int64_t K, const int32_t *rows, int64_t M, void *xq,
                                   float *xs, int mode, hipStream_t stream);
// The same dispatch from the token side: token row t (of x [T, K]) quantized
// once, written to rows dest[t * topk + k] of xq [M, K], xs [M, K/128] that
// lie in [0, M) (fp8bs_route.hip).
hipError_t launch_quant_act_scatter(const void *x, int64_t T, int64_t K, const int32_t *dest, int64_t topk,
                                    int64_t M, void *xq, float *xs, int mode, hipStream_t stream);
// The gated activation of gu [M, 2F] (gate columns first), rounded to bf16,
// then quantized 1x128: hq [M, F], hs [M, F/128] (fp8bs_swiglu.hip).
hipError_t launch_swiglu_quant(const void *gu, int64_t M, int64_t F, void *hq, float *hs, int mode,
                               hipStream_t stream);

// One weight tensor of a batched weight quantization (qt, st: the transposed
// codes [K, N] and scales [K/128, N/128], written by the dual launcher only).
struct WTensor {
    const void *w;
    void *q;
    float *s;
    int64_t N, K;
    void *qt = nullptr;
    float *st = nullptr;
};
// Quantizes `count` tensors (count >= 1, every N, K a positive multiple of
// 128) in as few launches as the kernel-argument budget allows.
hipError_t launch_quant_w(const WTensor *t, int64_t count, int mode, hipStream_t stream);
// The same, also writing each tensor's transposed codes and scales (qt, st).
hipError_t launch_quant_w_dual(const WTensor *t, int64_t count, int mode, hipStream_t stream);

// ---- GEMMs (fp8bs_gemm.hip) --------------------------------------------------

size_t gemm_workspace_size(int64_t M, int64_t N, int64_t K);
// pow2: every scale is a power of two (the kernels then apply the scales
// through the matrix cores' E8M0 operands where they can)
hipError_t launch_gemm(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                       int64_t K, void *y, int out_fp32, int pow2, void *workspace, hipStream_t stream);
// The product with per-row weight scales ws [N, K/128] (both operands in
// 1x128 blocks along K): the weight gradient.
hipError_t launch_gemm_1x128(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                             int64_t K, void *y, int out_fp32, int pow2, hipStream_t stream);
// Y = fp8_block_gemm(quant_act_1x128(x), Wq, Ws) from bf16 x; the workspace
// holds the quantized x (unless the shape runs fused) and the GEMM's own.
size_t linear_workspace_size(int64_t M, int64_t N, int64_t K);
hipError_t launch_linear(const void *x, const void *wq, const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                         int out_fp32, int pow2, void *workspace, hipStream_t stream);
// Y = fp8_block_gemm(...) (bf16, written to y unless y is null) together with
// quant_act_1x128(Y) into yq [M, N], ys [M, N/128]; mode is the scale mode of
// the operands and of the output's quantization.
size_t gemm_quant_workspace_size(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_quant(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                             int64_t K, void *y, void *yq, float *ys, int mode, void *workspace, hipStream_t stream);
// One activation row on the vector ALUs (fp8bs_gemv.hip): gemv_ok says
// whether the product qualifies (M == 1, K <= 16384); quantize 0 takes codes
// and scales, 1 / 2 bf16 activations quantized in-kernel (EXACT / POW2), with
// the codes and scale quant_act_1x128 writes.  No workspace.
bool gemv_ok(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemv(const void *x, const float *xs, const void *wq, const float *ws, int64_t N, int64_t K, void *y,
                       int out_fp32, int quantize, hipStream_t stream);
size_t grouped_workspace_size(int64_t E, int64_t M_total, int64_t N, int64_t K);
hipError_t launch_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                               const int32_t *offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void *y,
                               int out_fp32, int pow2, void *workspace, hipStream_t stream);
// Size of the library's static device array that stands in for the grouped
// workspace in fp8_block_grouped_gemm_noalloc, and its device address on the
// current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = (size_t)1 << 20;
hipError_t noalloc_scratch(void **ptr);

// ---- attention over an FP8 KV cache (fp8bs_attn.hip) -------------------------

// Hq / Hkv in {1, 2, 4, 8}
bool kv_attention_group_ok(int64_t Hq, int64_t Hkv);
size_t kv_attention_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv);
hipError_t launch_kv_attention(const void *q, const void *kq, const float *ks, const void *vq, const float *vs,
                               const int32_t *lens, int64_t B, int64_t T, int64_t Hq, int64_t Hkv, float sm_scale,
                               void *out, int out_fp32, void *workspace, hipStream_t stream);

} // namespace fp8bs
