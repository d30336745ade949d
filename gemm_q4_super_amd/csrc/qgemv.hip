// Fused quantize + GEMV entry points (q4k_quantize_gemv, q4k_quantize_gemv_batch):
// the streaming GEMV of stream_gemv.h with fp32 activations quantized to Q8
// inside the kernel, one launch per call.
#include "stream_gemv.h"

namespace q4k {

hipError_t launch_quantize_gemv_batch(const GemvProblem *probs, int count, int64_t K,
                                      int64_t M, hipStream_t stream) {
    const stream::Prepared none = {nullptr, nullptr, nullptr};
    return stream::run<true>(probs, count, K, M, none, stream);
}

hipError_t launch_quantize_gemv(const uint8_t *w, int64_t N, int64_t K, const float *x,
                                int64_t M, float *y, hipStream_t stream) {
    const GemvProblem p = {w, x, y, N};
    return launch_quantize_gemv_batch(&p, 1, K, M, stream);
}

}  // namespace q4k
