// bi_moe.h -- the batch-invariant MoE layer (host side).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "bi.h"

namespace bi {

size_t moe_workspace_size(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk);

// Byte offsets in the MoE workspace of the expert-sorted pair list, the bf16
// activations and the fp32 slot partials, and the total size (out[0..3]).
bi_status_t moe_layout_offsets(int64_t M, int64_t H, int64_t E, int64_t I, int64_t topk, int64_t* out);

bi_status_t moe_run(const uint16_t* x, const float* w_router, const float* b_router,
                    const uint16_t* w13, const uint16_t* w2, int64_t M, int64_t H, int64_t E,
                    int64_t I, int64_t topk, const bi_moe_options_t& opt, int32_t* topk_ids, float* topk_probs, float* y,
                    void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace bi
