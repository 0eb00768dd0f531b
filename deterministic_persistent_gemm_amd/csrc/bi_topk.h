// bi_topk.h -- deterministic per-row top-k of indexer scores (host side).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace bi {

// Longest row (columns) one workgroup holds: 1024 threads x 8 columns.
constexpr int64_t kTopkMaxCols = 8192;
// batches of at least this many rows use the 512-thread form (four rows per
// compute unit) instead of the 1024-thread form (two rows, shorter per row)
constexpr int64_t kTopkWideRows = 1024;

hipError_t launch_topk_rows(const float* scores, int64_t ld, int64_t rows, int64_t cols,
                            const int64_t* row_start, const int64_t* row_end, int64_t topk, int32_t* out,
                            int64_t ld_out, hipStream_t stream);

}  // namespace bi
