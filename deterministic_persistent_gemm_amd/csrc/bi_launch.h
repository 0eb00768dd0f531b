// bi_launch.h -- kernel launchers behind the C ABI (host side).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "bi.h"
#include "bi_plan.h"

namespace bi {

// How X is stored for an fp32-recipe call: fp32, or bf16 widened exactly to
// fp32 on load (the MoE router reads the layer's bf16 activations).
enum XKind { kXF32 = 0, kXBF16Widen = 1, kXBF16 = 2 };

struct LinearArgs {
    const void* x;
    int64_t ldx;
    const void* w;
    int64_t ldw;
    const float* bias;
    void* y;
    int y_bf16;
    int64_t ldy;
    int M, N, K;
};

// fold == false leaves a decode-path call with several k tiles at its tile
// partials (layout: [M tile][N tile][k tile][64 lanes] of f32x4 at ws +
// kDecodeCounterBytes) for a consumer that folds them itself in the same order.
hipError_t launch_linear(int xkind, const LinearArgs& a, const Plan& p, void* ws, hipStream_t s,
                         bool fold = true);

// bi_linear_f32 in two steps (bi_abi.cpp): the validation and the workspace
// bytes the automatic plan needs (nothing enqueued), and the call itself.
// no_split: the ring-fed fp32 tiles run unsplit (no workspace, same bits).
bi_status_t linear_f32_checked(const float* x, int64_t ldx, const float* w, int64_t ldw, const float* bias,
                               float* y, int64_t ldy, int64_t M, int64_t N, int64_t K, size_t* ws_needed,
                               bool no_split = false);
bi_status_t linear_f32_run(const float* x, int64_t ldx, const float* w, int64_t ldw, const float* bias, float* y,
                           int64_t ldy, int64_t M, int64_t N, int64_t K, void* ws, size_t ws_bytes,
                           hipStream_t stream, bool no_split = false);

// Diagnostic kernels (bi_lab.hip).
hipError_t launch_xcc_ids(uint32_t* out, int gx, int gy, hipStream_t s);
hipError_t launch_empty(int grid, int threads, hipStream_t s);
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, int grid, hipStream_t s);
hipError_t launch_clock(uint64_t* out, int grid, int iters, hipStream_t s);
hipError_t launch_lds_read(uint64_t* out, int grid, int iters, hipStream_t s);
hipError_t launch_l2_read(const void* src, int64_t bytes, int iters, uint32_t* sink, int grid, hipStream_t s);
hipError_t launch_mfma_rate(uint64_t* out, bool bf16, int chains, int grid, int iters, hipStream_t s);

}  // namespace bi
