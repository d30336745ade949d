// Fused quantize + GEMV entry points (q4k_quantize_gemv, q4k_quantize_gemv_batch):
// the streaming GEMV of stream_gemv.h with fp32 activations quantized to Q8
// inside the kernel, one launch per call.
#include <algorithm>

#include "stream_gemv.h"

namespace q4k {

// A launch shape exists for (M, K): the plan with 2-row groups, one row group
// per lane and the most columns per lane M allows keeps the waves within
// kWaves and the LDS (staged rows plus the 2-row block's terms) within the
// workgroup limit; every other shape needs more of one or the other.
bool stream_fits(int64_t M, int64_t K) {
    if (M < 1 || M > 8 || K < kQK || K % kQK != 0) return false;
    const int64_t nsb = K / kQK;
    const int units = M <= 2 ? 8 : M <= 4 ? 4 : M <= 6 ? 2 : 1;   // stream::max_units<M>()
    if (nsb > (int64_t)stream::kWaves * 4 * std::min(3, units)) return false;
    return stream::q8_bytes((int)M, (int)nsb) + stream::col_bytes((int)M, 2, (int)nsb) <=
           lds_limit();
}

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
