// fp8bs_abi.hip -- the extern "C" boundary declared in include/fp8bs.h.
//
// Checks every argument before touching the device, verifies once per device
// that it is a gfx950, and hands over to the kernel launchers.  Nothing here
// allocates, synchronizes or throws.
#include <atomic>
#include <string.h>

#include "fp8bs.h"
#include "fp8bs_internal.hpp"

namespace {

constexpr int kMaxDevices = 64;
// 0 = not yet queried, 1 = gfx950, 2 = other device
std::atomic<int> g_device_kind[kMaxDevices];

int check_device()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0)
        return FP8BS_UNSUPPORTED_DEVICE;
    if (dev < kMaxDevices) {
        const int k = g_device_kind[dev].load(std::memory_order_relaxed);
        if (k != 0)
            return k == 1 ? FP8BS_OK : FP8BS_UNSUPPORTED_DEVICE;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return FP8BS_UNSUPPORTED_DEVICE;
    const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    if (dev < kMaxDevices)
        g_device_kind[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok ? FP8BS_OK : FP8BS_UNSUPPORTED_DEVICE;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// A device tensor argument: null is allowed only when it holds no element.
bool tensor_ok(const void *p, int64_t elems, size_t align)
{
    if (elems == 0)
        return true;
    return p != nullptr && aligned(p, align);
}

// Largest extent any kernel indexes with 32-bit tile counters.
constexpr int64_t kMaxDim = (int64_t)1 << 31;

int status_of(hipError_t e) { return e == hipSuccess ? FP8BS_OK : FP8BS_HIP_ERROR; }

int check_quant(const void *x, int64_t R, int64_t K, const void *q, const float *s, int mode, bool rows_blocked)
{
    if (R < 0 || K <= 0 || (mode != FP8BS_SCALE_EXACT && mode != FP8BS_SCALE_POW2))
        return FP8BS_INVALID_ARG;
    if (K % 128 != 0 || (rows_blocked && R % 128 != 0))
        return FP8BS_UNSUPPORTED_SHAPE;
    // grid sizes stay below 2^31 workgroups: activation blocks / 64, weight blocks
    if (R >= kMaxDim || K >= kMaxDim || R * (K / 128) >= kMaxDim * 64 || (R / 128) * (K / 128) >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    const int64_t n = R * K;
    if (!tensor_ok(x, n, 16) || !tensor_ok(q, n, 16) || !tensor_ok(s, n, 4))
        return FP8BS_INVALID_ARG;
    return FP8BS_OK;
}

int check_gemm_shape(int64_t M, int64_t N, int64_t K, int out_dtype)
{
    if (M < 0 || N <= 0 || K <= 0 || (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_FP32))
        return FP8BS_INVALID_ARG;
    if (N % 128 != 0 || K % 128 != 0)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    // output tiles are counted in 32-bit integers (work units, grid sizes)
    if (((M + 127) / 128) * (N / 128) >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    return FP8BS_OK;
}

int check_gemm_common(const void *xq, const float *xs, const void *y, int64_t M, int64_t N, int64_t K, int out_dtype)
{
    const int st = check_gemm_shape(M, N, K, out_dtype);
    if (st != FP8BS_OK)
        return st;
    if (!tensor_ok(xq, M * K, 16) || !tensor_ok(xs, M * K, 4) || !tensor_ok(y, M * N, 16))
        return FP8BS_INVALID_ARG;
    return FP8BS_OK;
}

} // namespace

extern "C" {

int fp8bs_abi_version(void) { return FP8BS_ABI_VERSION; }

const char *fp8bs_status_string(int status)
{
    switch (status) {
    case FP8BS_OK:
        return "ok";
    case FP8BS_INVALID_ARG:
        return "invalid argument (null or misaligned pointer, negative size, unknown enum value)";
    case FP8BS_UNSUPPORTED_SHAPE:
        return "unsupported shape (K, or N where required, not a multiple of 128, or too large)";
    case FP8BS_UNSUPPORTED_DEVICE:
        return "unsupported device (the current HIP device is not a gfx950)";
    case FP8BS_WORKSPACE_TOO_SMALL:
        return "workspace too small";
    case FP8BS_HIP_ERROR:
        return "HIP runtime error at launch";
    case FP8BS_SCRATCH_TOO_SMALL:
        return "the problem needs more scratch than the library's static device buffer holds "
               "(fp8_block_grouped_gemm_noalloc: use fp8_block_grouped_gemm with a workspace)";
    default:
        return "unknown status";
    }
}

int quant_act_1x128(const void *x_bf16, int64_t M, int64_t K, void *xq, float *xs, int scale_mode, void *stream)
{
    int st = check_quant(x_bf16, M, K, xq, xs, scale_mode, false);
    if (st != FP8BS_OK)
        return st;
    if (M == 0)
        return FP8BS_OK;
    if ((st = check_device()) != FP8BS_OK)
        return st;
    return status_of(fp8bs::launch_quant_act(x_bf16, M, K, xq, xs, scale_mode, (hipStream_t)stream));
}

int quant_act_1x128_t(const void *x_bf16, int64_t M, int64_t K, void *xqt, float *xst, int scale_mode, void *stream)
{
    // X^T [K, M] in 1x128 blocks along M: M must be a multiple of 128 as well
    if (M < 0 || K <= 0 || (scale_mode != FP8BS_SCALE_EXACT && scale_mode != FP8BS_SCALE_POW2))
        return FP8BS_INVALID_ARG;
    if (M % 128 != 0 || K % 128 != 0 || (M / 128) * (K / 128) >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (M == 0)
        return FP8BS_OK;
    int st = check_quant(x_bf16, K, M, xqt, xst, scale_mode, false);
    if (st != FP8BS_OK)
        return st;
    if ((st = check_device()) != FP8BS_OK)
        return st;
    return status_of(fp8bs::launch_quant_act_t(x_bf16, M, K, xqt, xst, scale_mode, (hipStream_t)stream));
}

int quant_act_1x128_dual(const void *x_bf16, int64_t M, int64_t K, void *xq, float *xs, void *xqt, float *xst,
                         int scale_mode, void *stream)
{
    if (M < 0 || K <= 0 || (scale_mode != FP8BS_SCALE_EXACT && scale_mode != FP8BS_SCALE_POW2))
        return FP8BS_INVALID_ARG;
    if (M % 128 != 0 || K % 128 != 0 || (M / 128) * (K / 128) >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (M == 0)
        return FP8BS_OK;
    int st = check_quant(x_bf16, M, K, xq, xs, scale_mode, false);
    if (st != FP8BS_OK)
        return st;
    if (!tensor_ok(xqt, M * K, 16) || !tensor_ok(xst, M * K, 4))
        return FP8BS_INVALID_ARG;
    if ((st = check_device()) != FP8BS_OK)
        return st;
    return status_of(
        fp8bs::launch_quant_act_t(x_bf16, M, K, xqt, xst, scale_mode, (hipStream_t)stream, xq, xs));
}

int quant_act_1x128_gather(const void *x_bf16, int64_t T, int64_t K, const int32_t *rows, int64_t M, void *xq,
                           float *xs, int scale_mode, void *stream)
{
    if (T < 0 || M < 0 || K <= 0 || (scale_mode != FP8BS_SCALE_EXACT && scale_mode != FP8BS_SCALE_POW2))
        return FP8BS_INVALID_ARG;
    if (K % 128 != 0 || K >= kMaxDim || T >= kMaxDim || M >= kMaxDim || M * (K / 128) >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (M == 0)
        return FP8BS_OK;
    if (!tensor_ok(x_bf16, T * K, 16) || !tensor_ok(rows, M, 4) || !tensor_ok(xq, M * K, 16) ||
        !tensor_ok(xs, M * K, 4))
        return FP8BS_INVALID_ARG;
    int st = check_device();
    if (st != FP8BS_OK)
        return st;
    return status_of(
        fp8bs::launch_quant_act_gather(x_bf16, T, K, rows, M, xq, xs, scale_mode, (hipStream_t)stream));
}

int quant_act_1x128_scatter(const void *x_bf16, int64_t T, int64_t K, const int32_t *dest, int64_t topk, int64_t M,
                            void *xq, float *xs, int scale_mode, void *stream)
{
    if (T < 0 || M < 0 || K <= 0 || topk < 0 || (scale_mode != FP8BS_SCALE_EXACT && scale_mode != FP8BS_SCALE_POW2))
        return FP8BS_INVALID_ARG;
    if (K % 128 != 0 || K >= kMaxDim || T >= kMaxDim || M >= kMaxDim || topk >= kMaxDim ||
        T * (K / 128) >= kMaxDim || M * (K / 128) >= kMaxDim || T * topk >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (T == 0 || topk == 0 || M == 0)
        return FP8BS_OK;
    if (!tensor_ok(x_bf16, T * K, 16) || !tensor_ok(dest, T * topk, 4) || !tensor_ok(xq, M * K, 16) ||
        !tensor_ok(xs, M * K, 4))
        return FP8BS_INVALID_ARG;
    int st = check_device();
    if (st != FP8BS_OK)
        return st;
    return status_of(
        fp8bs::launch_quant_act_scatter(x_bf16, T, K, dest, topk, M, xq, xs, scale_mode, (hipStream_t)stream));
}

int swiglu_quant_1x128(const void *gu_bf16, int64_t M, int64_t F, void *hq, float *hs, int scale_mode, void *stream)
{
    if (M < 0 || F <= 0 || (scale_mode != FP8BS_SCALE_EXACT && scale_mode != FP8BS_SCALE_POW2))
        return FP8BS_INVALID_ARG;
    if (F % 128 != 0 || F >= kMaxDim || M >= kMaxDim || M * (F / 128) >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (M == 0)
        return FP8BS_OK;
    if (!tensor_ok(gu_bf16, 2 * M * F, 16) || !tensor_ok(hq, M * F, 16) || !tensor_ok(hs, M * F, 4))
        return FP8BS_INVALID_ARG;
    int st = check_device();
    if (st != FP8BS_OK)
        return st;
    return status_of(fp8bs::launch_swiglu_quant(gu_bf16, M, F, hq, hs, scale_mode, (hipStream_t)stream));
}

int quant_w_128x128(const void *w_bf16, int64_t N, int64_t K, void *wq, float *ws, int scale_mode, void *stream)
{
    int st = check_quant(w_bf16, N, K, wq, ws, scale_mode, true);
    if (st != FP8BS_OK)
        return st;
    if (N == 0)
        return FP8BS_OK;
    if ((st = check_device()) != FP8BS_OK)
        return st;
    fp8bs::WTensor t = {w_bf16, wq, ws, N, K};
    return status_of(fp8bs::launch_quant_w(&t, 1, scale_mode, (hipStream_t)stream));
}

int quant_w_128x128_batched(int64_t count, const void *const *w_bf16, const int64_t *N, const int64_t *K,
                            void *const *wq, float *const *ws, int scale_mode, void *stream)
{
    if (count < 0)
        return FP8BS_INVALID_ARG;
    if (count == 0)
        return FP8BS_OK;
    if (!w_bf16 || !N || !K || !wq || !ws)
        return FP8BS_INVALID_ARG;
    bool any = false;
    for (int64_t i = 0; i < count; ++i) {
        const int st = check_quant(w_bf16[i], N[i], K[i], wq[i], ws[i], scale_mode, true);
        if (st != FP8BS_OK)
            return st;
        any = any || N[i] > 0;
    }
    if (!any)
        return FP8BS_OK;
    int st = check_device();
    if (st != FP8BS_OK)
        return st;
    // pack the non-empty tensors, in order, a fixed-size batch at a time
    fp8bs::WTensor buf[64];
    int64_t n = 0;
    for (int64_t i = 0; i < count; ++i) {
        if (N[i] == 0)
            continue;
        buf[n++] = fp8bs::WTensor{w_bf16[i], wq[i], ws[i], N[i], K[i]};
        if (n == 64) {
            if (fp8bs::launch_quant_w(buf, n, scale_mode, (hipStream_t)stream) != hipSuccess)
                return FP8BS_HIP_ERROR;
            n = 0;
        }
    }
    if (n > 0 && fp8bs::launch_quant_w(buf, n, scale_mode, (hipStream_t)stream) != hipSuccess)
        return FP8BS_HIP_ERROR;
    return FP8BS_OK;
}

static int quant_w_dual_impl(int64_t count, const void *const *w_bf16, const int64_t *N, const int64_t *K,
                             void *const *wq, float *const *ws, void *const *wqt, float *const *wst, int scale_mode,
                             void *stream)
{
    if (count < 0)
        return FP8BS_INVALID_ARG;
    if (count == 0)
        return FP8BS_OK;
    if (!w_bf16 || !N || !K || !wq || !ws || !wqt || !wst)
        return FP8BS_INVALID_ARG;
    bool any = false;
    for (int64_t i = 0; i < count; ++i) {
        int st = check_quant(w_bf16[i], N[i], K[i], wq[i], ws[i], scale_mode, true);
        if (st != FP8BS_OK)
            return st;
        // the transposed outputs: codes [K, N] and scales [K/128, N/128]
        if (!tensor_ok(wqt[i], N[i] * K[i], 16) || !tensor_ok(wst[i], N[i] * K[i], 4))
            return FP8BS_INVALID_ARG;
        any = any || N[i] > 0;
    }
    if (!any)
        return FP8BS_OK;
    int st = check_device();
    if (st != FP8BS_OK)
        return st;
    fp8bs::WTensor buf[64];
    int64_t n = 0;
    for (int64_t i = 0; i < count; ++i) {
        if (N[i] == 0)
            continue;
        buf[n++] = fp8bs::WTensor{w_bf16[i], wq[i], ws[i], N[i], K[i], wqt[i], wst[i]};
        if (n == 64) {
            if (fp8bs::launch_quant_w_dual(buf, n, scale_mode, (hipStream_t)stream) != hipSuccess)
                return FP8BS_HIP_ERROR;
            n = 0;
        }
    }
    if (n > 0 && fp8bs::launch_quant_w_dual(buf, n, scale_mode, (hipStream_t)stream) != hipSuccess)
        return FP8BS_HIP_ERROR;
    return FP8BS_OK;
}

int quant_w_128x128_dual(const void *w_bf16, int64_t N, int64_t K, void *wq, float *ws, void *wqt, float *wst,
                         int scale_mode, void *stream)
{
    return quant_w_dual_impl(1, &w_bf16, &N, &K, &wq, &ws, &wqt, &wst, scale_mode, stream);
}

int quant_w_128x128_dual_batched(int64_t count, const void *const *w_bf16, const int64_t *N, const int64_t *K,
                                 void *const *wq, float *const *ws, void *const *wqt, float *const *wst,
                                 int scale_mode, void *stream)
{
    return quant_w_dual_impl(count, w_bf16, N, K, wq, ws, wqt, wst, scale_mode, stream);
}

static int gemm_1x128_impl(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                           int64_t K, void *y, int out_dtype, int pow2, void *stream)
{
    int st = check_gemm_common(xq, xs, y, M, N, K, out_dtype);
    if (st != FP8BS_OK)
        return st;
    // per-row weight scales: [N, K/128]
    if (!tensor_ok(wq, N * K, 16) || !tensor_ok(ws, N * K, 4))
        return FP8BS_INVALID_ARG;
    if (M == 0)
        return FP8BS_OK;
    if ((st = check_device()) != FP8BS_OK)
        return st;
    return status_of(fp8bs::launch_gemm_1x128(xq, xs, wq, ws, M, N, K, y, out_dtype == FP8BS_OUT_FP32, pow2,
                                              (hipStream_t)stream));
}

int fp8_block_gemm_1x128(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                         int64_t K, void *y, int out_dtype, void *stream)
{
    return gemm_1x128_impl(xq, xs, wq, ws, M, N, K, y, out_dtype, 0, stream);
}

int fp8_block_gemm_1x128_pow2(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                              int64_t K, void *y, int out_dtype, void *stream)
{
    return gemm_1x128_impl(xq, xs, wq, ws, M, N, K, y, out_dtype, 1, stream);
}

size_t fp8bs_gemm_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0)
        return 0;
    return fp8bs::gemm_workspace_size(M, N, K);
}

size_t fp8bs_grouped_workspace_size(int64_t E, int64_t M_total, int64_t N, int64_t K)
{
    if (E <= 0 || M_total <= 0 || N <= 0 || K <= 0)
        return 0;
    return fp8bs::grouped_workspace_size(E, M_total, N, K);
}

static int gemm_impl(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                     int64_t K, void *y, int out_dtype, int pow2, void *workspace, size_t workspace_bytes,
                     void *stream)
{
    int st = check_gemm_common(xq, xs, y, M, N, K, out_dtype);
    if (st != FP8BS_OK)
        return st;
    if (!tensor_ok(wq, N * K, 16) || !tensor_ok(ws, N * K, 4))
        return FP8BS_INVALID_ARG;
    if (M == 0)
        return FP8BS_OK;
    const size_t need = fp8bs::gemm_workspace_size(M, N, K);
    if (workspace_bytes < need)
        return FP8BS_WORKSPACE_TOO_SMALL;
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 16)))
        return FP8BS_INVALID_ARG;
    if ((st = check_device()) != FP8BS_OK)
        return st;
    // one activation row: the weight-streaming GEMV (any scales; it takes no workspace)
    if (fp8bs::gemv_ok(M, N, K))
        return status_of(fp8bs::launch_gemv(xq, xs, wq, ws, N, K, y, out_dtype == FP8BS_OUT_FP32, 0,
                                            (hipStream_t)stream));
    return status_of(fp8bs::launch_gemm(xq, xs, wq, ws, M, N, K, y, out_dtype == FP8BS_OUT_FP32, pow2, workspace,
                                        (hipStream_t)stream));
}

static int grouped_impl(const void *xq, const float *xs, const void *wq, const float *ws,
                        const int32_t *group_offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void *y,
                        int out_dtype, int pow2, void *workspace, size_t workspace_bytes, void *stream,
                        bool noalloc = false)
{
    int st = check_gemm_common(xq, xs, y, M_total, N, K, out_dtype);
    if (st != FP8BS_OK)
        return st;
    if (E < 0 || (E == 0 && M_total > 0) || E >= kMaxDim)
        return FP8BS_INVALID_ARG;
    if (M_total == 0)
        return FP8BS_OK;
    if (!tensor_ok(wq, E * N * K, 16) || !tensor_ok(ws, E * N * K, 4) || group_offsets == nullptr ||
        !aligned(group_offsets, 4))
        return FP8BS_INVALID_ARG;
    if ((M_total + 127) / 128 + E >= kMaxDim / (N / 128))
        return FP8BS_UNSUPPORTED_SHAPE;
    const size_t need = fp8bs::grouped_workspace_size(E, M_total, N, K);
    if (noalloc) {
        if (need > FP8BS_NOALLOC_SCRATCH_BYTES)
            return FP8BS_SCRATCH_TOO_SMALL;
    } else {
        if (workspace_bytes < need)
            return FP8BS_WORKSPACE_TOO_SMALL;
        if (need > 0 && (workspace == nullptr || !aligned(workspace, 16)))
            return FP8BS_INVALID_ARG;
    }
    if ((st = check_device()) != FP8BS_OK)
        return st;
    // the no-allocation form: the tables go to the library's static device array
    if (noalloc && need > 0 && fp8bs::noalloc_scratch(&workspace) != hipSuccess)
        return FP8BS_HIP_ERROR;
    return status_of(fp8bs::launch_grouped_gemm(xq, xs, wq, ws, group_offsets, E, M_total, N, K, y,
                                                out_dtype == FP8BS_OUT_FP32, pow2, workspace, (hipStream_t)stream));
}

static_assert(FP8BS_NOALLOC_SCRATCH_BYTES == fp8bs::kNoallocScratchBytes,
              "the header's scratch size must be the library's");

size_t fp8bs_linear_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0)
        return 0;
    return fp8bs::linear_workspace_size(M, N, K);
}

static int linear_impl(const void *x, const void *wq, const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                       int out_dtype, int pow2, void *workspace, size_t workspace_bytes, void *stream)
{
    // the GEMM's shape checks, the activation quantizer's grid limit, then
    // the pointers (x [M, K] bf16 takes the place of xq and xs)
    int st = check_gemm_shape(M, N, K, out_dtype);
    if (st != FP8BS_OK)
        return st;
    if (M * (K / 128) >= kMaxDim * 64)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (!tensor_ok(x, M * K, 16) || !tensor_ok(y, M * N, 16) || !tensor_ok(wq, N * K, 16) ||
        !tensor_ok(ws, N * K, 4))
        return FP8BS_INVALID_ARG;
    if (M == 0)
        return FP8BS_OK;
    const size_t need = fp8bs::linear_workspace_size(M, N, K);
    if (workspace_bytes < need)
        return FP8BS_WORKSPACE_TOO_SMALL;
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 16)))
        return FP8BS_INVALID_ARG;
    if ((st = check_device()) != FP8BS_OK)
        return st;
    // one activation row: the GEMV quantizes it in-kernel (the workspace goes unused)
    if (fp8bs::gemv_ok(M, N, K))
        return status_of(fp8bs::launch_gemv(x, nullptr, wq, ws, N, K, y, out_dtype == FP8BS_OUT_FP32, pow2 ? 2 : 1,
                                            (hipStream_t)stream));
    return status_of(fp8bs::launch_linear(x, wq, ws, M, N, K, y, out_dtype == FP8BS_OUT_FP32, pow2, workspace,
                                          (hipStream_t)stream));
}

int fp8_block_linear(const void *x_bf16, const void *wq, const float *ws, int64_t M, int64_t N, int64_t K, void *y,
                     int out_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return linear_impl(x_bf16, wq, ws, M, N, K, y, out_dtype, 0, workspace, workspace_bytes, stream);
}

int fp8_block_linear_pow2(const void *x_bf16, const void *wq, const float *ws, int64_t M, int64_t N, int64_t K,
                          void *y, int out_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return linear_impl(x_bf16, wq, ws, M, N, K, y, out_dtype, 1, workspace, workspace_bytes, stream);
}

int fp8_block_gemm(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N, int64_t K,
                   void *y, int out_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm_impl(xq, xs, wq, ws, M, N, K, y, out_dtype, 0, workspace, workspace_bytes, stream);
}

int fp8_block_gemm_pow2(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                        int64_t K, void *y, int out_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return gemm_impl(xq, xs, wq, ws, M, N, K, y, out_dtype, 1, workspace, workspace_bytes, stream);
}

int fp8_block_grouped_gemm(const void *xq, const float *xs, const void *wq, const float *ws,
                           const int32_t *group_offsets, int64_t E, int64_t M_total, int64_t N, int64_t K, void *y,
                           int out_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return grouped_impl(xq, xs, wq, ws, group_offsets, E, M_total, N, K, y, out_dtype, 0, workspace, workspace_bytes,
                        stream);
}

int fp8_block_grouped_gemm_pow2(const void *xq, const float *xs, const void *wq, const float *ws,
                                const int32_t *group_offsets, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                void *y, int out_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    return grouped_impl(xq, xs, wq, ws, group_offsets, E, M_total, N, K, y, out_dtype, 1, workspace, workspace_bytes,
                        stream);
}

int fp8_block_grouped_gemm_noalloc(const void *xq, const float *xs, const void *wq, const float *ws,
                                   const int32_t *group_offsets, int64_t E, int64_t M_total, int64_t N, int64_t K,
                                   void *y, int out_dtype, void *stream)
{
    return grouped_impl(xq, xs, wq, ws, group_offsets, E, M_total, N, K, y, out_dtype, 0, nullptr, 0, stream, true);
}

size_t fp8bs_gemm_quant_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0)
        return 0;
    return fp8bs::gemm_quant_workspace_size(M, N, K);
}

int fp8_block_gemm_quant(const void *xq, const float *xs, const void *wq, const float *ws, int64_t M, int64_t N,
                         int64_t K, void *y, void *yq, float *ys, int scale_mode, void *workspace,
                         size_t workspace_bytes, void *stream)
{
    if (scale_mode != FP8BS_SCALE_EXACT && scale_mode != FP8BS_SCALE_POW2)
        return FP8BS_INVALID_ARG;
    int st = check_gemm_shape(M, N, K, FP8BS_OUT_BF16);
    if (st != FP8BS_OK)
        return st;
    // the quantized output's scale grid [M, N/128] (as quant_act_1x128 of Y)
    if (M * (N / 128) >= kMaxDim * 64)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (!tensor_ok(xq, M * K, 16) || !tensor_ok(xs, M * K, 4) || !tensor_ok(wq, N * K, 16) ||
        !tensor_ok(ws, N * K, 4) || !tensor_ok(yq, M * N, 16) || !tensor_ok(ys, M * N, 4))
        return FP8BS_INVALID_ARG;
    if (y != nullptr && !aligned(y, 16))
        return FP8BS_INVALID_ARG;
    if (M == 0)
        return FP8BS_OK;
    const size_t need = fp8bs::gemm_quant_workspace_size(M, N, K);
    if (workspace_bytes < need)
        return FP8BS_WORKSPACE_TOO_SMALL;
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 16)))
        return FP8BS_INVALID_ARG;
    if ((st = check_device()) != FP8BS_OK)
        return st;
    return status_of(fp8bs::launch_gemm_quant(xq, xs, wq, ws, M, N, K, y, yq, ys, scale_mode, workspace,
                                              (hipStream_t)stream));
}

size_t fp8bs_kv_attention_workspace_size(int64_t B, int64_t T, int64_t Hq, int64_t Hkv)
{
    if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || !fp8bs::kv_attention_group_ok(Hq, Hkv))
        return 0;
    return fp8bs::kv_attention_workspace_size(B, T, Hq, Hkv);
}

int fp8_kv_attention_decode(const void *q_bf16, const void *kq, const float *ks, const void *vq, const float *vs,
                            const int32_t *lens, int64_t B, int64_t T, int64_t Hq, int64_t Hkv, float sm_scale,
                            void *out, int out_dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    if (B < 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || !(sm_scale == sm_scale) || sm_scale > 3.0e38f ||
        sm_scale < -3.0e38f || (out_dtype != FP8BS_OUT_BF16 && out_dtype != FP8BS_OUT_FP32))
        return FP8BS_INVALID_ARG;
    if (!fp8bs::kv_attention_group_ok(Hq, Hkv))
        return FP8BS_UNSUPPORTED_SHAPE;
    // 32-bit byte offsets within one sequence's cache rows (the kernel also
    // forms those of one tile past the end); workgroup counts
    if ((T + 128) * Hkv * 128 >= kMaxDim || B * Hkv >= kMaxDim || B * Hq >= kMaxDim)
        return FP8BS_UNSUPPORTED_SHAPE;
    if (B == 0)
        return FP8BS_OK;
    const int64_t cache = B * T * Hkv * 128;
    if (!tensor_ok(q_bf16, B * Hq * 128, 16) || !tensor_ok(kq, cache, 16) || !tensor_ok(vq, cache, 16) ||
        !tensor_ok(ks, cache, 4) || !tensor_ok(vs, cache, 4) || !tensor_ok(lens, B, 4) ||
        !tensor_ok(out, B * Hq * 128, 16))
        return FP8BS_INVALID_ARG;
    const size_t need = fp8bs::kv_attention_workspace_size(B, T, Hq, Hkv);
    if (workspace_bytes < need)
        return FP8BS_WORKSPACE_TOO_SMALL;
    if (need > 0 && (workspace == nullptr || !aligned(workspace, 16)))
        return FP8BS_INVALID_ARG;
    int st = check_device();
    if (st != FP8BS_OK)
        return st;
    return status_of(fp8bs::launch_kv_attention(q_bf16, kq, ks, vq, vs, lens, B, T, Hq, Hkv, sm_scale, out,
                                                out_dtype == FP8BS_OUT_FP32, workspace, (hipStream_t)stream));
}

} // extern "C"
