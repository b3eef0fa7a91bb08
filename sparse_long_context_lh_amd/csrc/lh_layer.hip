// The step on either side of the Lighthouse layer: the Q, K and V
// projections in, the layer's scatter-back out, and the backward through both
// to the input and the projection weights (aitrends summary, 방법론 item 5:
// gradients reach W_Q, W_K and W_V through scatter-back, the gather and the
// attention). The projections are plain dense GEMMs and run in rocBLAS
// (bf16 or fp32 operands, fp32 accumulation), on a workspace carved from the
// caller's ws and with atomics disallowed, so results are reproducible; the
// layer itself is lh_forward / lh_backward on the projected rows.
//
// Layouts (row-major): x [N][d_model]; W [d_model][3 H d], columns
// [Q heads 0..H-1 | K heads | V heads], d per head; the projected rows
// [3][H][N][d] in the layer's layout; out and dout [H][N][d]; dx [N][d_model];
// dW like W. Every GEMM is one large GEMM over all heads (Y = x W, dW =
// x^T dY, dx = dY W^T with Y and dY as [N][3 H d]); a copy kernel moves rows
// between [N][3 H d] and the layer's [3][H][N][d] (a strided-batched GEMM per
// head block writing the layer's layout directly ran at 0.6 of these GEMMs'
// rate).
#include <string.h>

#include <mutex>

#include <rocblas/rocblas.h>

#include "lh_device.h"
#include "lh_internal.h"

namespace lh {

constexpr size_t kBlasWorkspace = size_t(32) << 20; // handed to rocBLAS on every call
constexpr int kMaxBlasDevices = 64;

static std::mutex g_blas_mu; // guards the handles and each call's set_stream / set_workspace / gemm sequence
static rocblas_handle g_blas[kMaxBlasDevices];

// The current device's rocBLAS handle (created on the first call there).
static lh_status blas_handle(rocblas_handle *out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxBlasDevices)
        return LH_EHIP;
    if (!g_blas[dev]) {
        rocblas_handle h = nullptr;
        if (rocblas_create_handle(&h) != rocblas_status_success)
            return LH_EHIP;
        rocblas_set_atomics_mode(h, rocblas_atomics_not_allowed);
        g_blas[dev] = h;
    }
    *out = g_blas[dev];
    return LH_OK;
}

struct LayerPlan {
    Plan lh;
    int64_t N;
    int H, d, dm;
    size_t elem;                 // bytes per element
    size_t qkv_off, qkv_bytes;   // [3][H][N][d] projected rows (backward: reused for [N][3Hd] gradients)
    size_t lh_off;               // the layer's own workspace
    size_t blas_off;             // rocBLAS workspace
    size_t dqkv_off;             // [3][H][N][d] gradients at the projected rows (backward only)
    size_t total;
};

static size_t rup(size_t x) { return (x + 255) / 256 * 256; }

static lh_status layer_plan(int64_t N, int H, int d, int dm, int L, int p, int k, lh_dtype dt, LayerPlan *lp)
{
    memset(lp, 0, sizeof(*lp));
    lh_status st = make_plan(N, H, d, L, p, k, dt, &lp->lh);
    if (st != LH_OK)
        return st;
    if (dm < 1)
        return LH_EINVAL;
    if (dm % 8 != 0 || dm > 65536 || (int64_t)3 * H * d > (int64_t(1) << 30) || N > (int64_t(1) << 31) - 1)
        return LH_EUNSUPPORTED; // 16-byte rows; rocBLAS int sizes
    lp->N = N; lp->H = H; lp->d = d; lp->dm = dm;
    lp->elem = dt == LH_BF16 ? 2 : 4;
    lp->qkv_bytes = 3 * (size_t)H * (size_t)N * (size_t)d * lp->elem;
    lp->qkv_off = 0;
    lp->lh_off = rup(lp->qkv_bytes);
    lp->blas_off = lp->lh_off + rup(lp->lh.total);
    lp->dqkv_off = lp->blas_off + kBlasWorkspace;
    lp->total = lp->dqkv_off + rup(lp->qkv_bytes);
    if (lp->total > kMaxWorkspace)
        return LH_EUNSUPPORTED;
    return LH_OK;
}

static rocblas_datatype blas_type(lh_dtype dt) { return dt == LH_BF16 ? rocblas_datatype_bf16_r : rocblas_datatype_f32_r; }

// Rows between the layer's [3][H][N][d] ("heads") and [N][3 H d] ("rows",
// row n is token n at every projected column), 16 bytes per thread in the
// order of the rows layout (so one of the two sides is always contiguous).
template <typename T, bool TO_ROWS>
__global__ __launch_bounds__(256) void k_relayout(const T *__restrict__ src, T *__restrict__ dst, int64_t N, int HB,
                                                  int d)
{
    constexpr int V = 16 / sizeof(T);
    const int per_row = d / V; // 16-byte pieces of one head row
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t total = (int64_t)N * HB * per_row;
    if (i >= total)
        return;
    const int c = (int)(i % per_row);
    const int64_t rest = i / per_row;
    const int b = (int)(rest % HB); // head of the [3][H] block
    const int64_t n = rest / HB;
    const int64_t heads = ((int64_t)b * N + n) * d + c * V, rows = (n * HB + b) * d + c * V;
    const uint4 val = *reinterpret_cast<const uint4 *>(src + (TO_ROWS ? heads : rows));
    *reinterpret_cast<uint4 *>(dst + (TO_ROWS ? rows : heads)) = val;
}

static hipError_t launch_relayout(const void *src, void *dst, int64_t N, int HB, int d, lh_dtype dt, bool to_rows,
                                  hipStream_t s)
{
    const int V = dt == LH_BF16 ? 8 : 4;
    const int64_t total = N * HB * (d / V);
    const dim3 grid((unsigned)((total + 255) / 256));
    if (dt == LH_BF16) {
        if (to_rows)
            hipLaunchKernelGGL((k_relayout<uint16_t, true>), grid, dim3(256), 0, s, (const uint16_t *)src,
                               (uint16_t *)dst, N, HB, d);
        else
            hipLaunchKernelGGL((k_relayout<uint16_t, false>), grid, dim3(256), 0, s, (const uint16_t *)src,
                               (uint16_t *)dst, N, HB, d);
    } else {
        if (to_rows)
            hipLaunchKernelGGL((k_relayout<float, true>), grid, dim3(256), 0, s, (const float *)src, (float *)dst,
                               N, HB, d);
        else
            hipLaunchKernelGGL((k_relayout<float, false>), grid, dim3(256), 0, s, (const float *)src, (float *)dst,
                               N, HB, d);
    }
    return hipGetLastError();
}

} // namespace lh

using namespace lh;

extern "C" {

size_t lh_layer_workspace_bytes(int64_t N, int H, int d, int d_model, int L, int p, int k, lh_dtype dt)
{
    LayerPlan lp;
    if (layer_plan(N, H, d, d_model, L, p, k, dt, &lp) != LH_OK)
        return 0;
    return lp.total;
}

lh_status lh_layer_forward(const void *x, const void *w_qkv, int64_t N, int H, int d, int d_model, int L, int p,
                           int k_sel, lh_dtype dt, void *out, void *ws, size_t ws_bytes, void *stream)
{
    LayerPlan lp;
    lh_status st = layer_plan(N, H, d, d_model, L, p, k_sel, dt, &lp);
    if (st != LH_OK)
        return st;
    if (!x || !w_qkv || !out || ((uintptr_t)x & 15u) || ((uintptr_t)w_qkv & 15u) || ((uintptr_t)out & 15u))
        return LH_EINVAL;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < lp.total)
        return LH_EWORKSPACE;
    char *w = static_cast<char *>(ws);
    const hipStream_t s = (hipStream_t)stream;
    const int HB = 3 * H;
    {
        // Y = x W as [N][3Hd] in the (still free) gradient region; column-major:
        // Y^T (3Hd x N, ld 3Hd) = W^T (stored 3Hd x dm, ld 3Hd) . x^T (dm x N, ld dm)
        std::lock_guard<std::mutex> lock(g_blas_mu);
        rocblas_handle hb;
        if ((st = blas_handle(&hb)) != LH_OK)
            return st;
        const float one = 1.0f, zero = 0.0f;
        if (rocblas_set_stream(hb, s) != rocblas_status_success ||
            rocblas_set_workspace(hb, w + lp.blas_off, kBlasWorkspace) != rocblas_status_success)
            return LH_EHIP;
        const rocblas_datatype t = blas_type(dt);
        if (rocblas_gemm_ex(hb, rocblas_operation_none, rocblas_operation_none, HB * d, (int)N, d_model, &one, w_qkv,
                            t, HB * d, x, t, d_model, &zero, w + lp.dqkv_off, t, HB * d, w + lp.dqkv_off, t, HB * d,
                            rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
            return LH_EHIP;
    }
    if (launch_relayout(w + lp.dqkv_off, w + lp.qkv_off, N, HB, d, dt, false, s) != hipSuccess)
        return LH_EHIP;
    const size_t plane = (size_t)H * (size_t)N * (size_t)d * lp.elem;
    return lh_forward(w + lp.qkv_off, w + lp.qkv_off + plane, w + lp.qkv_off + 2 * plane, N, H, d, L, p, k_sel, dt,
                      out, w + lp.lh_off, lp.lh.total, stream);
}

lh_status lh_layer_backward(const void *x, const void *w_qkv, const void *dout, int64_t N, int H, int d, int d_model,
                            int L, int p, int k_sel, lh_dtype dt, void *dx, void *dw_qkv, void *ws, size_t ws_bytes,
                            void *stream)
{
    LayerPlan lp;
    lh_status st = layer_plan(N, H, d, d_model, L, p, k_sel, dt, &lp);
    if (st != LH_OK)
        return st;
    if (!x || !w_qkv || !dout || !dx || !dw_qkv || ((uintptr_t)x & 15u) || ((uintptr_t)w_qkv & 15u) ||
        ((uintptr_t)dout & 15u) || ((uintptr_t)dx & 15u) || ((uintptr_t)dw_qkv & 15u))
        return LH_EINVAL;
    if (!ws || ((uintptr_t)ws & 255u) || ws_bytes < lp.total)
        return LH_EWORKSPACE;
    char *w = static_cast<char *>(ws);
    const hipStream_t s = (hipStream_t)stream;
    const size_t plane = (size_t)H * (size_t)N * (size_t)d * lp.elem;
    char *dqkv = w + lp.dqkv_off;
    if ((st = lh_backward(dout, N, H, d, L, p, k_sel, dt, dqkv, dqkv + plane, dqkv + 2 * plane, w + lp.lh_off,
                          lp.lh.total, stream)) != LH_OK)
        return st;
    const int HB = 3 * H;
    // the projected rows are no longer needed: their place takes the
    // gradients as rows of 3 H d columns, the operand of dx's single GEMM
    if (launch_relayout(dqkv, w + lp.qkv_off, N, HB, d, dt, true, s) != hipSuccess)
        return LH_EHIP;
    std::lock_guard<std::mutex> lock(g_blas_mu);
    rocblas_handle hb;
    if ((st = blas_handle(&hb)) != LH_OK)
        return st;
    const float one = 1.0f, zero = 0.0f;
    if (rocblas_set_stream(hb, s) != rocblas_status_success ||
        rocblas_set_workspace(hb, w + lp.blas_off, kBlasWorkspace) != rocblas_status_success)
        return LH_EHIP;
    const rocblas_datatype t = blas_type(dt);
    // dW = x^T dY; column-major: dW^T (3Hd x dm, ld 3Hd) = dY^T (3Hd x N, ld 3Hd)
    // . x (N x dm: x^T stored dm x N, transposed)
    if (rocblas_gemm_ex(hb, rocblas_operation_none, rocblas_operation_transpose, HB * d, d_model, (int)N, &one,
                        w + lp.qkv_off, t, HB * d, x, t, d_model, &zero, dw_qkv, t, HB * d, dw_qkv, t, HB * d,
                        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
        return LH_EHIP;
    // dx = dX_rows [N][3Hd] . W^T; column-major: dx^T (dm x N, ld dm) =
    // W^T^T (W^T stored 3Hd x dm, transposed) . dX_rows^T (3Hd x N, ld 3Hd)
    if (rocblas_gemm_ex(hb, rocblas_operation_transpose, rocblas_operation_none, d_model, (int)N, HB * d, &one, w_qkv,
                        t, HB * d, w + lp.qkv_off, t, HB * d, &zero, dx, t, d_model, dx, t, d_model,
                        rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
        return LH_EHIP;
    return LH_OK;
}

} // extern "C"
