// Internal declarations shared by the libq4k.so translation units.
// Launchers validate nothing: the C-ABI layer in q4k_api.hip does that first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "../../include/q4k.h"

namespace q4k {

constexpr int kQK = 256;       // weights per Q4_K super-block
constexpr int kSB = 144;       // bytes per Q4_K super-block
constexpr int kQB = 32;        // Q8 block / Q4_K sub-block length

// Compute units of the current device (cached per device; 256 if unknown).
inline int cu_count() {
    static std::atomic<int> n[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = n[dev].load(std::memory_order_relaxed);
    if (!v) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        n[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

// LDS bytes one workgroup may allocate on the current device (cached per
// device; 65536 if unknown).
inline size_t lds_limit() {
    static std::atomic<int> n[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 65536;
    int v = n[dev].load(std::memory_order_relaxed);
    if (!v) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess ||
            v <= 0)
            v = 65536;
        n[dev].store(v, std::memory_order_relaxed);
    }
    return (size_t)v;
}

// Routed-expert limits (the route grouping runs in one workgroup's LDS).
constexpr int kMoeMaxPairs = 4096;     // T * topk
constexpr int kMoeMaxExperts = 4096;

hipError_t launch_quantize(const float *x, int64_t M, int64_t K, const float *gate,
                           int8_t *codes, float *scales, int32_t *sums,
                           hipStream_t stream);

hipError_t launch_gemv(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       hipStream_t stream);

// Small-batch GEMV on the matrix cores (prepared Q8 rows, M = 2..8), where its
// LDS holds the rows and scales / sums are 16-byte aligned; the same bits as
// the streaming GEMV.
bool gemv_mfma_fits(int64_t K, int64_t M, const void *scales, const void *sums);
// N: the rows of the launch (all its products').
bool gemv_mfma_preferred(int64_t N, int64_t K, int64_t M, const void *scales, const void *sums);
hipError_t launch_gemv_mfma(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                            const float *scales, const int32_t *sums, int64_t M, float *y,
                            hipStream_t stream);

// Q6_K GEMV on prepared Q8 rows or fp32 rows quantized inside (M <= 8,
// K <= kQ6MaxK, the staged rows within one workgroup's LDS: q6k_fits).
constexpr int64_t kQ6MaxK = 48 * 256;
bool q6k_fits(int64_t M, int64_t K);
hipError_t launch_q6k_gemv(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                           const float *scales, int64_t M, float *y, hipStream_t stream);
hipError_t launch_q6k_quantize_gemv(const uint8_t *w, int64_t N, int64_t K, const float *x,
                                    int64_t M, float *y, hipStream_t stream);

// Streaming GEMV (fused Q8 quantization or prepared rows): M <= 8 rows whose
// Q8 codes, scales and sums fit one workgroup's LDS with the smallest row block.
bool stream_fits(int64_t M, int64_t K);
hipError_t launch_quantize_gemv(const uint8_t *w, int64_t N, int64_t K, const float *x,
                                int64_t M, float *y, hipStream_t stream);
hipError_t launch_quantize_gemv_residual(const uint8_t *w, int64_t N, int64_t K, const float *x,
                                         int64_t M, const float *residual, float *y,
                                         hipStream_t stream);
using GemvProblem = q4k_gemv_problem;
// Q6_K GEMV over up to kMaxGemvBatch products (Q6_K weights in w), one launch:
// shared prepared Q8 rows, or fp32 rows per product (x) quantized inside.
hipError_t launch_q6k_gemv_batch(const GemvProblem *probs, int count, int64_t K,
                                 const int8_t *codes, const float *scales, int64_t M,
                                 hipStream_t stream);
hipError_t launch_q6k_quantize_gemv_batch(const GemvProblem *probs, int count, int64_t K,
                                          int64_t M, hipStream_t stream);
// Matrix-core GEMV over up to kMaxGemvBatch products with the same K and rows,
// one launch (the same bits as one launch per product).
hipError_t launch_gemv_mfma_batch(const GemvProblem *probs, int count, int64_t K,
                                  const int8_t *codes, const float *scales, const int32_t *sums,
                                  int64_t M, hipStream_t stream);
constexpr int kMaxGemvBatch = 8;
// The streaming GEMV over a batch on prepared Q8 rows (M <= 8, stream_fits):
// the kernel of q4k_gemv's streaming path, one launch.
hipError_t launch_gemv_batch_prepared(const GemvProblem *probs, int count, int64_t K,
                                      const int8_t *codes, const float *scales,
                                      const int32_t *sums, int64_t M, hipStream_t stream);
hipError_t launch_quantize_gemv_batch(const GemvProblem *probs, int count, int64_t K,
                                      int64_t M, hipStream_t stream);

// Prefill GEMM.  `workspace` (null, or gemm_workspace_bytes() bytes whose
// first kGemmCounters ints are zero) lets tiles be split across workgroups.
constexpr int kGemmCounters = 16384;   // split-tile counters (tiles x matrix-core waves)
constexpr int kGemmMaxGroups = 256;    // workgroups of a split launch
size_t gemm_workspace_bytes();
// The library's own GEMM scratch on the current device (a static device array
// of gemm_static_scratch_bytes() bytes; null if it cannot be resolved), and a
// launch that zeroes the counters at the start of a workspace.
void *gemm_static_scratch();
size_t gemm_static_scratch_bytes();
hipError_t launch_clear_counters(void *workspace, hipStream_t stream);
hipError_t launch_gemm(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       void *workspace, hipStream_t stream);
using GemmProblem = q4k_gemm_problem;
constexpr int kMaxGemmBatch = 8;
hipError_t launch_gemm_batch(const GemmProblem *probs, int count, int64_t K,
                             const int8_t *codes, const float *scales, const int32_t *sums,
                             int64_t M, void *workspace, hipStream_t stream);

hipError_t launch_q6k_gemm_batch(const GemmProblem *probs, int count, int64_t K,
                                 const int8_t *codes, const float *scales, int64_t M,
                                 void *workspace, hipStream_t stream);

size_t moe_workspace_bytes(int64_t T, int64_t topk, int64_t n_experts, int64_t N);

hipError_t launch_moe_gemv(const uint8_t *w, int64_t n_experts, int64_t stride,
                           int64_t N, int64_t K, const int32_t *ids, const float *route_w,
                           int64_t T, int64_t topk, const int8_t *codes,
                           const float *scales, const int32_t *sums, int act_per_slot,
                           float *y, void *workspace, hipStream_t stream);

size_t moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t H, int64_t F);

hipError_t launch_moe_ffn(const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                          int64_t n_experts, int64_t stride_gu, int64_t stride_down, int64_t H,
                          int64_t F, const int32_t *ids, const float *route_w, int64_t T,
                          int64_t topk, const float *x, float *y, void *workspace,
                          hipStream_t stream);

// INT8 KV cache and decode attention (head_dim 128).
constexpr int kAttnHeadDim = 128;
constexpr int kAttnMaxM = 8;           // query tokens per call
constexpr int kAttnMaxGroup = 8;       // query heads per kv head
constexpr int kAttnMaxKvHeads = 64;
constexpr int kMaxAttnChunks = 32;     // position chunks per (kv head, query block)
constexpr int kAttnTargetGroups = 256; // workgroups the chunking aims at
constexpr size_t kAttnCounterBytes = 4096;   // one counter per (kv head, query block)

size_t attn_workspace_bytes(int64_t M, int64_t n_head, int64_t n_kv);

hipError_t launch_kv_store(const float *k, const float *v, int64_t M, int64_t n_kv, int64_t pos0,
                           int64_t cap, int8_t *kc, float *ks, int8_t *vc, float *vs,
                           hipStream_t stream);

hipError_t launch_attn(const float *q, int64_t M, int64_t n_head, int64_t n_kv, const int8_t *kc,
                       const float *ks, const int8_t *vc, const float *vs, int64_t cap,
                       int64_t n_ctx, float scale, float *out, void *workspace,
                       hipStream_t stream);

// Measurement aids (not on the product path).
hipError_t launch_stream_read(const void *buf, int64_t bytes, int64_t grid, unsigned *sink,
                              hipStream_t stream);
hipError_t launch_empty(int64_t grid, hipStream_t stream);
hipError_t launch_mfma_valu(int64_t grid, int64_t iters, int vrep, int what, float *sink,
                            hipStream_t stream);

}  // namespace q4k
