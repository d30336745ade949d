// Quantize + GEMV with the residual add in the last step
// (q4k_quantize_gemv_residual): y = residual + Q8(x) W^T, the decode step's
// update of the residual stream by the attention-output and down projections
// ("genie-ai-runtime ...", section 4, Path C, which folds that add into the
// GEMV).  The streaming GEMV of stream_gemv.h with its residual switch on; the
// product is formed exactly as in q4k_quantize_gemv.  Its own translation unit
// so that these kernel instances compile beside the others.
#include "stream_gemv.h"

namespace q4k {

hipError_t launch_quantize_gemv_residual(const uint8_t *w, int64_t N, int64_t K, const float *x,
                                         int64_t M, const float *residual, float *y,
                                         hipStream_t stream) {
    const GemvProblem p = {w, x, y, N};
    const stream::Prepared Q = {nullptr, nullptr, nullptr, residual};
    return stream::run<true, true>(&p, 1, K, M, Q, stream);
}

}  // namespace q4k
