// Routed-expert grouped GEMV (placeholder).
#include "q4k_internal.h"

namespace q4k {
size_t moe_workspace_bytes(int64_t, int64_t, int64_t) { return 256; }
hipError_t launch_moe_gemv(const uint8_t *, int64_t, int64_t, int64_t, int64_t, const int32_t *,
                           const float *, int64_t, int64_t, const int8_t *, const float *,
                           const int32_t *, int, float *, void *, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace q4k
