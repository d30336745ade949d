// C-ABI entry points of libq4k.so (declared in include/q4k.h).
// Every argument is checked here, on the host, before anything is launched.
#include <math.h>

#include "../../include/q4k.h"
#include "q4k_internal.h"

namespace {

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int from_hip(hipError_t e) {
    if (e == hipErrorNotSupported) return Q4K_ENOTIMPL;
    return e == hipSuccess ? Q4K_OK : Q4K_EHIP;
}

// Sizes beyond these would overflow the 32-bit grid/index arithmetic of the
// kernels; far above any projection of the models in scope.
constexpr int64_t kMaxDim = int64_t(1) << 24;

int check_matrix_args(const void *w, int64_t N, int64_t K, const int8_t *codes,
                      const float *scales, const int32_t *sums, int64_t M, float *y) {
    if (!w || !codes || !scales || !sums || !y) return Q4K_EINVAL;
    if (N < 1 || K < q4k::kQK || K % q4k::kQK != 0 || M < 1) return Q4K_ESHAPE;
    if (N > kMaxDim || K > kMaxDim || M > kMaxDim) return Q4K_ESHAPE;
    if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(sums, 4) ||
        !aligned(y, 4))
        return Q4K_EALIGN;
    return Q4K_OK;
}

}  // namespace

extern "C" {

int q4k_quantize_act(const float *x, int64_t M, int64_t K, const float *gate, int8_t *codes,
                     float *scales, int32_t *sums, void *stream) {
    if (!x || !codes || !scales || !sums) return Q4K_EINVAL;
    if (M < 1 || K < q4k::kQB || K % q4k::kQB != 0) return Q4K_ESHAPE;
    if (M > kMaxDim || K > kMaxDim || M * (K / q4k::kQB) > (int64_t(1) << 36)) return Q4K_ESHAPE;
    if (!aligned(x, 16) || !aligned(codes, 16) || (gate && !aligned(gate, 16)) ||
        !aligned(scales, 4) || !aligned(sums, 4))
        return Q4K_EALIGN;
    return from_hip(q4k::launch_quantize(x, M, K, gate, codes, scales, sums,
                                         static_cast<hipStream_t>(stream)));
}

int q4k_gemv(const void *w, int64_t N, int64_t K, const int8_t *codes, const float *scales,
             const int32_t *sums, int64_t M, float *y, void *stream) {
    int st = check_matrix_args(w, N, K, codes, scales, sums, M, y);
    if (st != Q4K_OK) return st;
    if (M > 8) return Q4K_ESHAPE;
    return from_hip(q4k::launch_gemv(static_cast<const uint8_t *>(w), N, K, codes, scales,
                                     sums, M, y, static_cast<hipStream_t>(stream)));
}

int q4k_quantize_gemv(const void *w, int64_t N, int64_t K, const float *x, int64_t M,
                      float *y, void *stream) {
    if (!w || !x || !y) return Q4K_EINVAL;
    if (N < 1 || K < q4k::kQK || K % q4k::kQK != 0 || M < 1 || M > 8) return Q4K_ESHAPE;
    if (N > kMaxDim || K > kMaxDim || !q4k::stream_fits(M, K)) return Q4K_ESHAPE;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4K_EALIGN;
    return from_hip(q4k::launch_quantize_gemv(static_cast<const uint8_t *>(w), N, K, x, M, y,
                                              static_cast<hipStream_t>(stream)));
}

int q4k_quantize_gemv_residual(const void *w, int64_t N, int64_t K, const float *x,
                               int64_t M, const float *residual, float *y, void *stream) {
    if (!w || !x || !y || !residual) return Q4K_EINVAL;
    if (N < 1 || K < q4k::kQK || K % q4k::kQK != 0 || M < 1 || M > 8) return Q4K_ESHAPE;
    if (N > kMaxDim || K > kMaxDim || !q4k::stream_fits(M, K)) return Q4K_ESHAPE;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4) || !aligned(residual, 4))
        return Q4K_EALIGN;
    // In place (residual == y) or disjoint: a partial overlap would read
    // elements another thread has already written.
    const uintptr_t ry = reinterpret_cast<uintptr_t>(y), rr = reinterpret_cast<uintptr_t>(residual);
    const uintptr_t n = static_cast<uintptr_t>(M * N) * sizeof(float);
    if (ry != rr && ry < rr + n && rr < ry + n) return Q4K_EINVAL;
    return from_hip(q4k::launch_quantize_gemv_residual(static_cast<const uint8_t *>(w), N, K, x, M,
                                                       residual, y,
                                                       static_cast<hipStream_t>(stream)));
}

int q4k_quantize_gemv_batch(const q4k_gemv_problem *problems, int count, int64_t K,
                            int64_t M, void *stream) {
    if (!problems) return Q4K_EINVAL;
    if (count < 1 || count > q4k::kMaxGemvBatch) return Q4K_ESHAPE;
    if (K < q4k::kQK || K % q4k::kQK != 0 || K > kMaxDim || M < 1 || M > 8 ||
        !q4k::stream_fits(M, K))
        return Q4K_ESHAPE;
    for (int i = 0; i < count; ++i) {
        const q4k_gemv_problem &p = problems[i];
        if (!p.w || !p.x || !p.y) return Q4K_EINVAL;
        if (p.N < 1 || p.N > kMaxDim) return Q4K_ESHAPE;
        if (!aligned(p.w, 16) || !aligned(p.x, 16) || !aligned(p.y, 4)) return Q4K_EALIGN;
    }
    return from_hip(q4k::launch_quantize_gemv_batch(problems, count, K, M,
                                                    static_cast<hipStream_t>(stream)));
}

// A workspace is optional (null with 0 bytes); when given it must be large
// enough and 256-byte aligned.
static int check_gemm_workspace(const void *workspace, size_t workspace_bytes) {
    if (!workspace) return workspace_bytes == 0 ? Q4K_OK : Q4K_EWORKSPACE;
    if (workspace_bytes < q4k::gemm_workspace_bytes()) return Q4K_EWORKSPACE;
    if (!aligned(workspace, 256)) return Q4K_EALIGN;
    return Q4K_OK;
}

size_t q4k_gemm_workspace_bytes(void) { return q4k::gemm_workspace_bytes(); }

int q4k_gemm(const void *w, int64_t N, int64_t K, const int8_t *codes, const float *scales,
             const int32_t *sums, int64_t M, float *y, void *workspace, size_t workspace_bytes,
             void *stream) {
    int st = check_matrix_args(w, N, K, codes, scales, sums, M, y);
    if (st != Q4K_OK) return st;
    st = check_gemm_workspace(workspace, workspace_bytes);
    if (st != Q4K_OK) return st;
    return from_hip(q4k::launch_gemm(static_cast<const uint8_t *>(w), N, K, codes, scales,
                                     sums, M, y, workspace, static_cast<hipStream_t>(stream)));
}

int q4k_gemm_batch(const q4k_gemm_problem *problems, int count, int64_t K, const int8_t *codes,
                   const float *scales, const int32_t *sums, int64_t M, void *workspace,
                   size_t workspace_bytes, void *stream) {
    if (!problems) return Q4K_EINVAL;
    if (count < 1 || count > q4k::kMaxGemmBatch) return Q4K_ESHAPE;
    for (int i = 0; i < count; ++i) {
        const q4k_gemm_problem &p = problems[i];
        int st = check_matrix_args(p.w, p.N, K, codes, scales, sums, M, p.y);
        if (st != Q4K_OK) return st;
    }
    int st = check_gemm_workspace(workspace, workspace_bytes);
    if (st != Q4K_OK) return st;
    return from_hip(q4k::launch_gemm_batch(problems, count, K, codes, scales, sums, M, workspace,
                                           static_cast<hipStream_t>(stream)));
}

int q4k_gemm_batch_noalloc(const q4k_gemm_problem *problems, int count, int64_t K,
                           const int8_t *codes, const float *scales, const int32_t *sums,
                           int64_t M, void *stream) {
    if (!problems) return Q4K_EINVAL;
    if (count < 1 || count > q4k::kMaxGemmBatch) return Q4K_ESHAPE;
    for (int i = 0; i < count; ++i) {
        const q4k_gemm_problem &p = problems[i];
        int st = check_matrix_args(p.w, p.N, K, codes, scales, sums, M, p.y);
        if (st != Q4K_OK) return st;
    }
    if (q4k::gemm_static_scratch_bytes() < q4k::gemm_workspace_bytes()) return Q4K_EWORKSPACE;
    void *ws = q4k::gemm_static_scratch();
    if (!ws) return Q4K_EHIP;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = q4k::launch_clear_counters(ws, s);
    if (e != hipSuccess) return from_hip(e);
    return from_hip(q4k::launch_gemm_batch(problems, count, K, codes, scales, sums, M, ws, s));
}

size_t q4k_moe_workspace_bytes(int64_t T, int64_t topk, int64_t n_experts, int64_t N) {
    if (T < 1 || topk < 1 || n_experts < 1 || topk > n_experts ||
        T * topk > q4k::kMoeMaxPairs || n_experts > q4k::kMoeMaxExperts || N < 1 || N > kMaxDim)
        return 0;
    return q4k::moe_workspace_bytes(T, topk, n_experts, N);
}

int q4k_moe_gemv(const void *w_experts, int64_t n_experts, int64_t expert_stride_bytes,
                 int64_t N, int64_t K, const int32_t *ids, const float *route_w, int64_t T,
                 int64_t topk, const int8_t *codes, const float *scales, const int32_t *sums,
                 int act_per_slot, float *y, void *workspace, size_t workspace_bytes,
                 void *stream) {
    if (!w_experts || !ids || !codes || !scales || !sums || !y) return Q4K_EINVAL;
    if (act_per_slot != 0 && act_per_slot != 1) return Q4K_EINVAL;
    if (N < 1 || K < q4k::kQK || K % q4k::kQK != 0 || N > kMaxDim || K > kMaxDim)
        return Q4K_ESHAPE;
    if (n_experts < 1 || n_experts > q4k::kMoeMaxExperts || T < 1 || topk < 1 ||
        topk > n_experts || T * topk > q4k::kMoeMaxPairs)
        return Q4K_ESHAPE;
    if (expert_stride_bytes < N * (K / q4k::kQK) * q4k::kSB || expert_stride_bytes % 16 != 0)
        return Q4K_ESHAPE;
    if (!aligned(w_experts, 16) || !aligned(codes, 16) || !aligned(scales, 4) ||
        !aligned(sums, 4) || !aligned(y, 4) || !aligned(ids, 4) ||
        (route_w && !aligned(route_w, 4)))
        return Q4K_EALIGN;
    const size_t need = q4k::moe_workspace_bytes(T, topk, n_experts, N);
    if (!workspace || workspace_bytes < need) return Q4K_EWORKSPACE;
    if (!aligned(workspace, 256)) return Q4K_EALIGN;
    return from_hip(q4k::launch_moe_gemv(static_cast<const uint8_t *>(w_experts), n_experts,
                                         expert_stride_bytes, N, K, ids, route_w, T, topk,
                                         codes, scales, sums, act_per_slot, y, workspace,
                                         static_cast<hipStream_t>(stream)));
}

size_t q4k_moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t n_experts, int64_t H,
                                   int64_t F) {
    if (T < 1 || topk < 1 || n_experts < 1 || topk > n_experts ||
        T * topk > q4k::kMoeMaxPairs || n_experts > q4k::kMoeMaxExperts || H < 1 ||
        H > kMaxDim || F < 1 || F > kMaxDim)
        return 0;
    return q4k::moe_ffn_workspace_bytes(T, topk, H, F);
}

int q4k_moe_ffn(const void *w_gate, const void *w_up, const void *w_down, int64_t n_experts,
                int64_t stride_gate_up, int64_t stride_down, int64_t H, int64_t F,
                const int32_t *ids, const float *route_w, int64_t T, int64_t topk,
                const float *x, float *y, void *workspace, size_t workspace_bytes,
                void *stream) {
    if (!w_gate || !w_up || !w_down || !ids || !route_w || !x || !y) return Q4K_EINVAL;
    if (H < q4k::kQK || H % q4k::kQK != 0 || F < q4k::kQK || F % q4k::kQK != 0 ||
        H > kMaxDim || F > kMaxDim)
        return Q4K_ESHAPE;
    if (n_experts < 1 || n_experts > q4k::kMoeMaxExperts || T < 1 || topk < 1 ||
        topk > n_experts || T * topk > q4k::kMoeMaxPairs)
        return Q4K_ESHAPE;
    if (stride_gate_up < F * (H / q4k::kQK) * q4k::kSB || stride_gate_up % 16 != 0 ||
        stride_down < H * (F / q4k::kQK) * q4k::kSB || stride_down % 16 != 0)
        return Q4K_ESHAPE;
    if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16) ||
        !aligned(x, 16) || !aligned(y, 4) || !aligned(ids, 4) || !aligned(route_w, 4))
        return Q4K_EALIGN;
    const size_t need = q4k::moe_ffn_workspace_bytes(T, topk, H, F);
    if (!workspace || workspace_bytes < need) return Q4K_EWORKSPACE;
    if (!aligned(workspace, 256)) return Q4K_EALIGN;
    return from_hip(q4k::launch_moe_ffn(
        static_cast<const uint8_t *>(w_gate), static_cast<const uint8_t *>(w_up),
        static_cast<const uint8_t *>(w_down), n_experts, stride_gate_up, stride_down, H, F, ids,
        route_w, T, topk, x, y, workspace, static_cast<hipStream_t>(stream)));
}

int q6k_gemv(const void *w, int64_t N, int64_t K, const int8_t *codes, const float *scales,
             int64_t M, float *y, void *stream) {
    if (!w || !codes || !scales || !y) return Q4K_EINVAL;
    if (N < 1 || N > kMaxDim || K < q4k::kQK || K % q4k::kQK != 0 || K > q4k::kQ6MaxK ||
        M < 1 || M > 8 || !q4k::q6k_fits(M, K))
        return Q4K_ESHAPE;
    if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(y, 4))
        return Q4K_EALIGN;
    return from_hip(q4k::launch_q6k_gemv(static_cast<const uint8_t *>(w), N, K, codes, scales,
                                         M, y, static_cast<hipStream_t>(stream)));
}

int q6k_quantize_gemv(const void *w, int64_t N, int64_t K, const float *x, int64_t M, float *y,
                      void *stream) {
    if (!w || !x || !y) return Q4K_EINVAL;
    if (N < 1 || N > kMaxDim || K < q4k::kQK || K % q4k::kQK != 0 || K > q4k::kQ6MaxK ||
        M < 1 || M > 8 || !q4k::q6k_fits(M, K))
        return Q4K_ESHAPE;
    if (!aligned(w, 16) || !aligned(x, 16) || !aligned(y, 4)) return Q4K_EALIGN;
    return from_hip(q4k::launch_q6k_quantize_gemv(static_cast<const uint8_t *>(w), N, K, x, M, y,
                                                  static_cast<hipStream_t>(stream)));
}

int q6k_gemv_batch(const q4k_gemv_problem *problems, int count, int64_t K, const int8_t *codes,
                   const float *scales, int64_t M, void *stream) {
    if (!problems || !codes || !scales) return Q4K_EINVAL;
    if (count < 1 || count > q4k::kMaxGemvBatch) return Q4K_ESHAPE;
    if (K < q4k::kQK || K % q4k::kQK != 0 || K > q4k::kQ6MaxK || M < 1 || M > 8 ||
        !q4k::q6k_fits(M, K))
        return Q4K_ESHAPE;
    if (!aligned(codes, 16) || !aligned(scales, 4)) return Q4K_EALIGN;
    for (int i = 0; i < count; ++i) {
        const q4k_gemv_problem &p = problems[i];
        if (!p.w || !p.y) return Q4K_EINVAL;
        if (p.N < 1 || p.N > kMaxDim) return Q4K_ESHAPE;
        if (!aligned(p.w, 16) || !aligned(p.y, 4)) return Q4K_EALIGN;
    }
    return from_hip(q4k::launch_q6k_gemv_batch(problems, count, K, codes, scales, M,
                                               static_cast<hipStream_t>(stream)));
}

int q6k_quantize_gemv_batch(const q4k_gemv_problem *problems, int count, int64_t K, int64_t M,
                            void *stream) {
    if (!problems) return Q4K_EINVAL;
    if (count < 1 || count > q4k::kMaxGemvBatch) return Q4K_ESHAPE;
    if (K < q4k::kQK || K % q4k::kQK != 0 || K > q4k::kQ6MaxK || M < 1 || M > 8 ||
        !q4k::q6k_fits(M, K))
        return Q4K_ESHAPE;
    for (int i = 0; i < count; ++i) {
        const q4k_gemv_problem &p = problems[i];
        if (!p.w || !p.x || !p.y) return Q4K_EINVAL;
        if (p.N < 1 || p.N > kMaxDim) return Q4K_ESHAPE;
        if (!aligned(p.w, 16) || !aligned(p.x, 16) || !aligned(p.y, 4)) return Q4K_EALIGN;
    }
    return from_hip(q4k::launch_q6k_quantize_gemv_batch(problems, count, K, M,
                                                        static_cast<hipStream_t>(stream)));
}

int q6k_gemm(const void *w, int64_t N, int64_t K, const int8_t *codes, const float *scales,
             int64_t M, float *y, void *workspace, size_t workspace_bytes, void *stream) {
    if (!w || !codes || !scales || !y) return Q4K_EINVAL;
    if (N < 1 || K < q4k::kQK || K % q4k::kQK != 0 || M < 1) return Q4K_ESHAPE;
    if (N > kMaxDim || K > kMaxDim || M > kMaxDim) return Q4K_ESHAPE;
    if (!aligned(w, 16) || !aligned(codes, 16) || !aligned(scales, 4) || !aligned(y, 4))
        return Q4K_EALIGN;
    const int st = check_gemm_workspace(workspace, workspace_bytes);
    if (st != Q4K_OK) return st;
    const q4k::GemmProblem p = {w, y, N};
    return from_hip(q4k::launch_q6k_gemm_batch(&p, 1, K, codes, scales, M, workspace,
                                               static_cast<hipStream_t>(stream)));
}

int q4k_kv_store(const float *k, const float *v, int64_t M, int64_t n_kv, int64_t head_dim,
                 int64_t pos0, int64_t cap, int8_t *k_codes, float *k_scales, int8_t *v_codes,
                 float *v_scales, void *stream) {
    if (!k || !v || !k_codes || !k_scales || !v_codes || !v_scales) return Q4K_EINVAL;
    if (head_dim != q4k::kAttnHeadDim || M < 1 || M > 4096 || n_kv < 1 ||
        n_kv > q4k::kAttnMaxKvHeads || pos0 < 0 || cap > (int64_t(1) << 24) || pos0 + M > cap)
        return Q4K_ESHAPE;
    if (!aligned(k, 8) || !aligned(v, 8) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
        !aligned(k_scales, 4) || !aligned(v_scales, 4))
        return Q4K_EALIGN;
    return from_hip(q4k::launch_kv_store(k, v, M, n_kv, pos0, cap, k_codes, k_scales, v_codes,
                                         v_scales, static_cast<hipStream_t>(stream)));
}

size_t q4k_attn_workspace_bytes(int64_t M, int64_t n_head, int64_t n_kv) {
    if (M < 1 || n_kv < 1 || n_head < n_kv || n_head % n_kv != 0) return 0;
    return q4k::attn_workspace_bytes(M, n_head, n_kv);
}

int q4k_attn_decode(const float *q, int64_t M, int64_t n_head, int64_t n_kv, int64_t head_dim,
                    const int8_t *k_codes, const float *k_scales, const int8_t *v_codes,
                    const float *v_scales, int64_t cap, int64_t n_ctx, float scale, float *out,
                    void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !out) return Q4K_EINVAL;
    if (!(scale == scale) || scale == INFINITY || scale == -INFINITY) return Q4K_EINVAL;
    if (head_dim != q4k::kAttnHeadDim || M < 1 || M > q4k::kAttnMaxM || n_kv < 1 ||
        n_kv > q4k::kAttnMaxKvHeads || n_head < n_kv || n_head % n_kv != 0 ||
        n_head / n_kv > q4k::kAttnMaxGroup || n_ctx < M || n_ctx > cap ||
        cap > (int64_t(1) << 24))
        return Q4K_ESHAPE;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
        !aligned(k_scales, 4) || !aligned(v_scales, 4))
        return Q4K_EALIGN;
    if (!workspace || workspace_bytes < q4k::attn_workspace_bytes(M, n_head, n_kv))
        return Q4K_EWORKSPACE;
    if (!aligned(workspace, 256)) return Q4K_EALIGN;
    return from_hip(q4k::launch_attn(q, M, n_head, n_kv, k_codes, k_scales, v_codes, v_scales,
                                     cap, n_ctx, scale, out, workspace,
                                     static_cast<hipStream_t>(stream)));
}

int q4k_ceiling_stream_read(const void *buf, int64_t bytes, int64_t grid, unsigned *sink,
                            void *stream) {
    if (!buf || !sink) return Q4K_EINVAL;
    if (bytes < 16 || bytes % 16 != 0 || grid < 1 || grid > (int64_t(1) << 20)) return Q4K_ESHAPE;
    if (!aligned(buf, 16) || !aligned(sink, 4)) return Q4K_EALIGN;
    return from_hip(q4k::launch_stream_read(buf, bytes, grid, sink, static_cast<hipStream_t>(stream)));
}

int q4k_ceiling_empty(int64_t grid, void *stream) {
    if (grid < 1 || grid > (int64_t(1) << 20)) return Q4K_ESHAPE;
    return from_hip(q4k::launch_empty(grid, static_cast<hipStream_t>(stream)));
}

int q4k_ceiling_mfma_valu(int64_t grid, int64_t iters, int vrep, int what, float *sink,
                          void *stream) {
    if (!sink) return Q4K_EINVAL;
    if (grid < 1 || grid > (int64_t(1) << 20) || iters < 1 || iters > (int64_t(1) << 24) ||
        vrep < 0 || vrep > 64 || what < 1 || what > 3)
        return Q4K_ESHAPE;
    if (!aligned(sink, 4)) return Q4K_EALIGN;
    return from_hip(q4k::launch_mfma_valu(grid, iters, vrep, what, sink,
                                          static_cast<hipStream_t>(stream)));
}

const char *q4k_status_string(int status) {
    switch (status) {
    case Q4K_OK: return "ok";
    case Q4K_EINVAL: return "invalid argument (null pointer or bad value)";
    case Q4K_EALIGN: return "buffer not aligned as required";
    case Q4K_ESHAPE: return "size out of range";
    case Q4K_EWORKSPACE: return "workspace missing or too small";
    case Q4K_EHIP: return "HIP runtime error at launch";
    case Q4K_ENOTIMPL: return "operation not available in this build";
    default: return "unknown status";
    }
}

}  // extern "C"
