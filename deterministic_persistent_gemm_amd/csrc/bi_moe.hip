// bi_moe.hip -- batch-invariant MoE layer (placeholder until the kernels land).
#include <hip/hip_runtime.h>

#include "bi_moe.h"

namespace bi {

size_t moe_workspace_size(int64_t, int64_t, int64_t, int64_t, int64_t) { return 0; }

bi_status_t moe_run(const uint16_t*, const float*, const float*, const uint16_t*, const uint16_t*,
                    int64_t, int64_t, int64_t, int64_t, int64_t, int32_t*, float*, float*, void*,
                    size_t, hipStream_t)
{
    return BI_EUNSUPPORTED;
}

}  // namespace bi
