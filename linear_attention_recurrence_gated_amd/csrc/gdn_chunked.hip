// gdn_chunked.hip -- chunkwise-parallel prefill (placeholder until the kernels land).
#include "gdn_launch.h"

namespace gdn {

size_t prefill_chunked_workspace_bytes(int64_t, int64_t, int) { return 0; }

hipError_t launch_prefill_chunked(const void *, const void *, const void *, const float *, const float *,
                                  const int32_t *, const int32_t *, int64_t, int64_t, int, const float *, float *,
                                  float *, void *, hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace gdn
