// Prefill GEMM (placeholder until the matrix-core kernel lands).
#include "q4k_internal.h"

namespace q4k {
hipError_t launch_gemm(const uint8_t *, int64_t, int64_t, const int8_t *, const float *,
                       const int32_t *, int64_t, float *, hipStream_t) {
    return hipErrorNotSupported;
}
}  // namespace q4k
