// bi_abi.cpp -- the C ABI: argument validation, planning, launch.
//
// Every check happens on the host before anything is enqueued, and a rejected
// call enqueues nothing.  There is no fallback: a shape the recipe table cannot
// serve is an error, never a silent switch to a batch-dependent route (sparse
// MLA page, "Review follow-up" and the fail-closed commit: a batch-dependent
// result is raised, not returned).
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "bi.h"
#include "bi_launch.h"
#include "bi_moe.h"
#include "bi_plan.h"
#include "bi_topk.h"

using namespace bi;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Common validation of a linear call.  elem_x / elem_w: bytes per element.
bi_status_t check_linear(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias,
                         const void* y, int64_t ldy, int64_t M, int64_t N, int64_t K, int elem_x,
                         int elem_w, int elem_y)
{
    if (M < 0 || N < 0 || K < 0)
        return BI_EINVAL;
    if (M == 0)
        return BI_OK;
    if (!x || !w || !y)
        return BI_EINVAL;
    if (!aligned16(x) || !aligned16(w) || (bias && !aligned16(bias)) || !aligned16(y))
        return BI_EINVAL;
    if (ldx < K || ldw < K || ldy < N)
        return BI_EINVAL;
    if ((ldx * elem_x) % 16 != 0 || (ldw * elem_w) % 16 != 0 || (ldy * elem_y) % 4 != 0)
        return BI_EINVAL;
    if (M > (int64_t(1) << 30))
        return BI_EUNSUPPORTED;
    return BI_OK;
}

bi_status_t run_linear(int xkind, const void* x, int64_t ldx, const void* w, int64_t ldw,
                       const float* bias, void* y, int y_bf16, int64_t ldy, int64_t M, int64_t N,
                       int64_t K, const bi_recipe_t& recipe, int32_t path, void* ws, size_t ws_bytes,
                       hipStream_t stream)
{
    Plan p;
    bi_status_t st = make_plan(recipe, path, M, N, K, &p);
    if (st != BI_OK)
        return st;
    if (p.ws_bytes > 0 && (!ws || ws_bytes < p.ws_bytes || !aligned16(ws)))
        return BI_EWORKSPACE;
    LinearArgs a{x, ldx, w, ldw, bias, y, y_bf16, ldy, (int)M, (int)N, (int)K};
    return launch_linear(xkind, a, p, ws, stream) == hipSuccess ? BI_OK : BI_EHIP;
}

}  // namespace

namespace bi {

bi_status_t linear_f32_checked(const float* x, int64_t ldx, const float* w, int64_t ldw, const float* bias,
                               float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, size_t* ws_needed,
                               bool no_split)
{
    bi_status_t st = check_linear(x, ldx, w, ldw, bias, y, ldy, M, N, K, 4, 4, 4);
    if (st != BI_OK || M == 0) {
        *ws_needed = 0;
        return st;
    }
    bi_recipe_t r;
    if ((st = recipe_for(BI_F32, N, K, &r)) != BI_OK)
        return st;
    Plan p;
    if ((st = make_plan(r, BI_PATH_AUTO | (no_split ? kPathNoSplit : 0), M, N, K, &p)) != BI_OK)
        return st;
    *ws_needed = p.ws_bytes;
    return BI_OK;
}

bi_status_t linear_f32_run(const float* x, int64_t ldx, const float* w, int64_t ldw, const float* bias, float* y,
                           int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                           hipStream_t stream, bool no_split)
{
    bi_status_t st = check_linear(x, ldx, w, ldw, bias, y, ldy, M, N, K, 4, 4, 4);
    if (st != BI_OK || M == 0)
        return st;
    bi_recipe_t r;
    if ((st = recipe_for(BI_F32, N, K, &r)) != BI_OK)
        return st;
    return run_linear(kXF32, x, ldx, w, ldw, bias, y, 0, ldy, M, N, K, r,
                      BI_PATH_AUTO | (no_split ? kPathNoSplit : 0), ws, ws_bytes, stream);
}

}  // namespace bi

extern "C" {

const char* bi_status_str(bi_status_t s)
{
    switch (s) {
    case BI_OK: return "BI_OK";
    case BI_EINVAL: return "BI_EINVAL: invalid argument";
    case BI_EUNSUPPORTED: return "BI_EUNSUPPORTED: (dtype, N, K) not served by the recipe table";
    case BI_EWORKSPACE: return "BI_EWORKSPACE: workspace missing or too small";
    case BI_EHIP: return "BI_EHIP: HIP launch failed";
    }
    return "unknown bi_status_t";
}

bi_status_t bi_describe_recipe(int32_t dtype, int64_t N, int64_t K, bi_recipe_t* out)
{
    return recipe_for(dtype, N, K, out);
}

size_t bi_linear_workspace_size(int32_t dtype, int64_t M, int64_t N, int64_t K)
{
    bi_recipe_t r;
    if (recipe_for(dtype, N, K, &r) != BI_OK || M <= 0)
        return 0;
    Plan p;
    if (make_plan(r, BI_PATH_AUTO, M, N, K, &p) != BI_OK)
        return 0;
    return p.ws_bytes;
}

size_t bi_lab_workspace_size(const bi_recipe_t* recipe, int32_t path, int64_t M, int64_t N, int64_t K)
{
    if (!recipe || M <= 0)
        return 0;
    Plan p;
    if (make_plan(*recipe, path, M, N, K, &p) != BI_OK)
        return 0;
    return p.ws_bytes;
}

bi_status_t bi_linear_f32(const float* x, int64_t ldx, const float* w, int64_t ldw, const float* bias,
                          float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws,
                          size_t ws_bytes, hipStream_t stream)
{
    return linear_f32_run(x, ldx, w, ldw, bias, y, ldy, M, N, K, ws, ws_bytes, stream);
}

bi_status_t bi_linear_bf16(const uint16_t* x, int64_t ldx, const uint16_t* w, int64_t ldw,
                           const float* bias, void* y, int32_t y_dtype, int64_t ldy, int64_t M,
                           int64_t N, int64_t K, void* ws, size_t ws_bytes, hipStream_t stream)
{
    if (y_dtype != BI_F32 && y_dtype != BI_BF16)
        return BI_EINVAL;
    bi_status_t st = check_linear(x, ldx, w, ldw, bias, y, ldy, M, N, K, 2, 2, y_dtype == BI_BF16 ? 2 : 4);
    if (st != BI_OK || M == 0)
        return st;
    bi_recipe_t r;
    if ((st = recipe_for(BI_BF16, N, K, &r)) != BI_OK)
        return st;
    return run_linear(kXBF16, x, ldx, w, ldw, bias, y, y_dtype == BI_BF16, ldy, M, N, K, r, BI_PATH_AUTO,
                      ws, ws_bytes, stream);
}

bi_status_t bi_lab_linear(const void* x, int64_t ldx, const void* w, int64_t ldw, const float* bias,
                          void* y, int32_t y_dtype, int64_t ldy, int64_t M, int64_t N, int64_t K,
                          const bi_recipe_t* recipe, int32_t path, void* ws, size_t ws_bytes,
                          hipStream_t stream)
{
    if (!recipe || (y_dtype != BI_F32 && y_dtype != BI_BF16))
        return BI_EINVAL;
    const int ex = recipe->dtype == BI_F32 ? 4 : 2;
    bi_status_t st = check_linear(x, ldx, w, ldw, bias, y, ldy, M, N, K, ex, ex, y_dtype == BI_BF16 ? 2 : 4);
    if (st != BI_OK || M == 0)
        return st;
    return run_linear(recipe->dtype == BI_F32 ? kXF32 : kXBF16, x, ldx, w, ldw, bias, y,
                      y_dtype == BI_BF16, ldy, M, N, K, *recipe, path, ws, ws_bytes, stream);
}

bi_status_t bi_negctl_linear_f32(const float* x, int64_t ldx, const float* w, int64_t ldw,
                                 const float* bias, float* y, int64_t ldy, int64_t M, int64_t N,
                                 int64_t K, void* ws, size_t ws_bytes, hipStream_t stream)
{
    bi_status_t st = check_linear(x, ldx, w, ldw, bias, y, ldy, M, N, K, 4, 4, 4);
    if (st != BI_OK || M == 0)
        return st;
    bi_recipe_t r;
    if ((st = recipe_for(BI_F32, N, K, &r)) != BI_OK)
        return st;
    // the deliberate defect: the k tile width follows the batch size (never
    // wider than the shipped recipe's workspace needs)
    r.block_k = (M < 64) ? 2 * r.block_k : r.block_k;
    if (K % r.block_k != 0)
        return BI_EUNSUPPORTED;
    return run_linear(kXF32, x, ldx, w, ldw, bias, y, 0, ldy, M, N, K, r, BI_PATH_AUTO, ws, ws_bytes,
                      stream);
}

bi_status_t bi_lab_xcc_ids(uint32_t* out, int32_t grid_x, int32_t grid_y, hipStream_t stream)
{
    if (!out || grid_x <= 0 || grid_y <= 0 || (reinterpret_cast<uintptr_t>(out) & 3u) != 0)
        return BI_EINVAL;
    if ((int64_t)grid_x * grid_y > (int64_t(1) << 24) || grid_y > 65535)
        return BI_EUNSUPPORTED;
    return launch_xcc_ids(out, grid_x, grid_y, stream) == hipSuccess ? BI_OK : BI_EHIP;
}

bi_status_t bi_lab_plan(int32_t dtype, int64_t M, int64_t N, int64_t K, int32_t* path)
{
    if (!path || M <= 0)
        return BI_EINVAL;
    bi_recipe_t r;
    bi_status_t st = recipe_for(dtype, N, K, &r);
    if (st != BI_OK)
        return st;
    Plan p;
    if ((st = make_plan(r, BI_PATH_AUTO, M, N, K, &p)) != BI_OK)
        return st;
    *path = p.path;
    return BI_OK;
}

bi_status_t bi_lab_moe_layout(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk, int64_t* offsets)
{
    return moe_layout_offsets(M, H, E, I, topk, offsets);
}

bi_status_t bi_lab_empty(int32_t grid, int32_t threads, hipStream_t stream)
{
    if (grid <= 0 || threads <= 0 || threads > 1024 || threads % 64 != 0)
        return BI_EINVAL;
    return launch_empty(grid, threads, stream) == hipSuccess ? BI_OK : BI_EHIP;
}

bi_status_t bi_lab_stream_read(const void* src, int64_t bytes, uint32_t* sink, int32_t grid, hipStream_t stream)
{
    if (!src || !sink || bytes <= 0 || bytes % 16 != 0 || grid <= 0 || grid > 65535 ||
        (reinterpret_cast<uintptr_t>(src) & 15u) != 0 || (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return BI_EINVAL;
    return launch_stream_read(src, bytes, sink, grid, stream) == hipSuccess ? BI_OK : BI_EHIP;
}

bi_status_t bi_lab_l2_read(const void* src, int64_t bytes, int32_t iters, uint32_t* sink, int32_t grid,
                           hipStream_t stream)
{
    // a power of two of at least one full round (256 lanes x 8 loads x 16 B)
    // and at most 2 MiB
    if (!src || !sink || bytes < 32768 || bytes > (int64_t(2) << 20) || (bytes & (bytes - 1)) != 0 ||
        iters <= 0 || grid <= 0 || grid > 65535 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0 ||
        (reinterpret_cast<uintptr_t>(sink) & 3u) != 0)
        return BI_EINVAL;
    return launch_l2_read(src, bytes, iters, sink, grid, stream) == hipSuccess ? BI_OK : BI_EHIP;
}

bi_status_t bi_lab_clock(uint64_t* out, int32_t grid, int32_t iters, hipStream_t stream)
{
    if (!out || grid <= 0 || grid > 65535 || iters <= 0 || (reinterpret_cast<uintptr_t>(out) & 7u) != 0)
        return BI_EINVAL;
    return launch_clock(out, grid, iters, stream) == hipSuccess ? BI_OK : BI_EHIP;
}

bi_status_t bi_lab_lds_read(uint64_t* out, int32_t grid, int32_t iters, hipStream_t stream)
{
    if (!out || grid <= 0 || grid > 65535 || iters <= 0 || (reinterpret_cast<uintptr_t>(out) & 7u) != 0)
        return BI_EINVAL;
    return launch_lds_read(out, grid, iters, stream) == hipSuccess ? BI_OK : BI_EHIP;
}

bi_status_t bi_lab_mfma_rate(uint64_t* out, int32_t dtype, int32_t chains, int32_t grid, int32_t iters,
                             hipStream_t stream)
{
    if (!out || (dtype != BI_F32 && dtype != BI_BF16) || (chains != 1 && chains != 2 && chains != 4 && chains != 8) ||
        grid <= 0 || grid > 65535 || iters <= 0 || (reinterpret_cast<uintptr_t>(out) & 7u) != 0)
        return BI_EINVAL;
    return launch_mfma_rate(out, dtype == BI_BF16, chains, grid, iters, stream) == hipSuccess ? BI_OK : BI_EHIP;
}

size_t bi_moe_workspace_size(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk)
{
    return moe_workspace_size(M, H, E, I, topk);
}

bi_status_t bi_moe_grouped_gemm(const uint16_t* x, const float* w_router, const float* b_router,
                                const uint16_t* w13, const uint16_t* w2, int64_t M, int64_t H,
                                int64_t E, int64_t I, int64_t topk, int32_t* topk_ids,
                                float* topk_probs, float* y, void* ws, size_t ws_bytes,
                                hipStream_t stream)
{
    const bi_moe_options_t opt{BI_ACT_SWIGLU, 1, 0, 1};
    return moe_run(x, w_router, b_router, w13, w2, M, H, E, I, topk, opt, topk_ids, topk_probs, y, ws,
                   ws_bytes, stream);
}

bi_status_t bi_moe_grouped_gemm_ex(const uint16_t* x, const float* w_router, const float* b_router,
                                   const uint16_t* w1, const uint16_t* w2, int64_t M, int64_t H, int64_t E,
                                   int64_t I, int64_t topk, const bi_moe_options_t* options,
                                   int32_t* topk_ids, float* topk_probs, float* y, void* ws, size_t ws_bytes,
                                   hipStream_t stream)
{
    const bi_moe_options_t opt = options ? *options : bi_moe_options_t{BI_ACT_SWIGLU, 1, 0, 1};
    return moe_run(x, w_router, b_router, w1, w2, M, H, E, I, topk, opt, topk_ids, topk_probs, y, ws,
                   ws_bytes, stream);
}

bi_status_t bi_indexer_topk(const float* scores, int64_t ld, int64_t rows, int64_t cols,
                            const int64_t* row_start, const int64_t* row_end, int64_t topk,
                            int32_t* out, int64_t ld_out, hipStream_t stream)
{
    auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; };
    if (rows < 0 || cols < 0 || topk <= 0 || ld < cols || ld_out < topk)
        return BI_EINVAL;
    if (rows == 0)
        return BI_OK;
    if (cols > kTopkMaxCols || rows > (int64_t(1) << 31) - 1 || topk > (int64_t(1) << 30))
        return BI_EUNSUPPORTED;
    if (!out || (cols > 0 && !scores))
        return BI_EINVAL;
    if (!al(scores, 4) || !al(out, 4) || !al(row_start, 8) || !al(row_end, 8))
        return BI_EINVAL;
    return launch_topk_rows(scores, ld, rows, cols, row_start, row_end, topk, out, ld_out, stream) == hipSuccess
               ? BI_OK
               : BI_EHIP;
}

}  // extern "C"
