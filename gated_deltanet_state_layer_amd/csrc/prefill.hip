// Chunked prefill (placeholder until the kernels land).
#include "gdn_common.h"

namespace gdn {

size_t prefill_workspace_bytes(const gdn_pool*, int32_t, int64_t, int32_t) { return 0; }

hipError_t launch_prefill(const gdn_pool*, int32_t, int32_t, const int32_t*, const int32_t*,
                          int64_t, int32_t, const void*, const void*, const void*, const float*,
                          const float*, const float*, void*, void*, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace gdn
