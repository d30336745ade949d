/*
 * q4k.h -- C ABI of libq4k.so: Q4_K-weight x Q8-activation matrix products on
 * one AMD Instinct MI355X (gfx950).
 *
 * Source of the operations: the matrix products of edge LLM inference against
 * Q4_K_M-quantized weights described in "genie-ai-runtime: a Jetson edge LLM
 * inference engine that beats llama.cpp -- designing for unified memory":
 * batch-1 decode streams every weight once and is bandwidth-bound (section 2,
 * "The target hardware (and the roofline that dictates strategy)"); prefill is
 * a compute-bound batched product over all prompt tokens (section 3, Path B
 * and Path E); verification of several drafted tokens shares one weight read
 * (section 2 and section 9, speculative decoding).  The routed-expert product
 * follows the mixture-of-experts layers of "I'm making LLMs work on small and
 * old devices" (intro, expert pager; "Lessons").
 *
 * Formats (the pages name Q4_K_M but print no bytes; the public GGUF Q4_K
 * layout is used):
 *   Q4_K matrix W, N rows x K columns, K % 256 == 0: row-major, each row is
 *     K/256 super-blocks of 144 bytes: fp16 d, fp16 dmin, 12 bytes of 6-bit
 *     sub-block scales sc[8] and mins mn[8], 128 bytes of 4-bit quants q;
 *     weight = d*sc[j]*q - dmin*mn[j], j = (column % 256) / 32.
 *   Q8 activations, M rows x K: codes int8 [M][K] (row-major), scales fp32
 *     [M][K/32], sums int32 [M][K/32].  Per block of 32 values:
 *     scale = fl32(max|x| / 127), code = clamp(round-half-even(fl32(x/scale)),
 *     -127, 127), sum = sum of codes; an all-zero block has scale 0, codes 0.
 *   Products: y[m][n] = sum_k W[n][k] * scale[m][k/32] * code[m][k], i.e.
 *     y = x W^T, fp32 [M][N] row-major.
 *
 * Conventions for every call:
 *   - Pointers named as device buffers are device pointers on the current HIP
 *     device.  The caller owns every buffer; the library never allocates,
 *     frees, synchronizes, changes device or keeps state between calls.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     asynchronously on it; results are visible after the stream is synced.
 *   - Inputs are read-only; outputs are fully overwritten (never accumulated).
 *     The one input that may share memory with the output is the residual of
 *     q4k_quantize_gemv_residual (an in-place update of the residual stream).
 *   - Arguments are checked on the host before anything is launched; a failed
 *     check returns a negative status and launches nothing.  A launch error
 *     reported by the runtime returns Q4K_EHIP.  Nothing is printed and no
 *     C++ exception crosses the ABI.
 *   - Any N >= 1 and M >= 1 (within a call's limits) runs on the same fast
 *     kernels, with masked tails: there is no slower fallback for odd sizes.
 */
#ifndef Q4K_H
#define Q4K_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum q4k_status {
    Q4K_OK = 0,
    Q4K_EINVAL = -1,     /* null pointer or invalid value                    */
    Q4K_EALIGN = -2,     /* a buffer is not aligned as required              */
    Q4K_ESHAPE = -3,     /* size out of range (K % 256, M range, topk, ...)  */
    Q4K_EWORKSPACE = -4, /* workspace missing or too small                   */
    Q4K_EHIP = -5,       /* the HIP runtime reported an error at launch      */
    Q4K_ENOTIMPL = -6    /* operation not available in this build            */
};

/* Quantize M rows of K fp32 values (K % 32 == 0, M >= 1) to Q8 blocks of 32.
 *   x      device fp32 [M][K], 16-byte aligned.
 *   gate   NULL, or device fp32 [M][K]: then the value quantized is the SwiGLU
 *          h = silu(gate) * x = gate / (1 + exp(-gate)) * x, evaluated in fp64
 *          from the fp32 inputs and rounded once to fp32 (the pages name no
 *          activation function; SwiGLU is this library's reading for the
 *          routed-expert layer).  16-byte aligned.
 *   codes  device int8 [M][K], 16-byte aligned.
 *   scales device fp32 [M][K/32];  sums  device int32 [M][K/32].
 * Codes and sums are bit-exact with the definition above; non-finite inputs
 * are outside the contract (no fault, unspecified codes). */
int q4k_quantize_act(const float *x, int64_t M, int64_t K, const float *gate,
                     int8_t *codes, float *scales, int32_t *sums, void *stream);

/* Decode / small-batch GEMV: y[M][N] = Q8(x)[M][K] * W^T for M = 1..8
 * (batch-1 decode and the verification of up to 8 drafted tokens, which
 * shares one read of W).  Bandwidth-bound: W is streamed once with 16-byte
 * loads; for several rows on wide products the integer sub-block dots run on
 * the matrix cores (same result bits as the vector kernel, which runs
 * otherwise, e.g. when scales / sums are not 16-byte aligned).
 *   w       device Q4_K bytes, N rows x (K/256)*144 bytes, 16-byte aligned.
 *   N >= 1, K % 256 == 0, K >= 256, 1 <= M <= 8.
 *   codes   device int8 [M][K] (16-byte aligned); scales fp32 [M][K/32];
 *   sums    int32 [M][K/32]   -- as written by q4k_quantize_act.
 *   y       device fp32 [M][N].
 * fp32 result; accumulation order differs from the plain definition, within a
 * relative error of 2e-3 (absolute 1e-4 near zero). */
int q4k_gemv(const void *w, int64_t N, int64_t K, const int8_t *codes,
             const float *scales, const int32_t *sums, int64_t M, float *y,
             void *stream);

/* Quantize-and-GEMV in one launch: y[M][N] = Q8(x)[M][K] * W^T for fp32
 * activations x (device, [M][K], 16-byte aligned).  Each workgroup quantizes
 * the Q8 blocks it needs with the same arithmetic as q4k_quantize_act (codes
 * bit-identical), so the result equals q4k_quantize_act followed by q4k_gemv,
 * bit for bit, with one launch instead of two.  Limits: 1 <= M <= 8, and the
 * Q8 form of the M rows lives in one workgroup's LDS: M*(K/256)*328 bytes at
 * most the device's LDS per workgroup (163840 on MI355X: K up to 15872 at
 * M = 8, 31744 at M = 4, e.g. the 9728-wide down projection at any M), and
 * K/256 <= 192 (M <= 4), 128 (M <= 6), 64 (M <= 8).  Other arguments as for
 * q4k_gemv. */
int q4k_quantize_gemv(const void *w, int64_t N, int64_t K, const float *x,
                      int64_t M, float *y, void *stream);

/* Quantize-and-GEMV with the residual add in its last step:
 * y[M][N] = residual[M][N] + Q8(x)[M][K] * W^T.  The decode step adds the
 * output of the attention-output and down projections to the residual stream;
 * the genie page (section 4, Path C) folds that add into the GEMV, and
 * (section 6) keeps this single-kernel form over a split-K GEMV.  The product
 * is the one q4k_quantize_gemv computes, bit for bit, and the add is one fp32
 * rounding per element, so y equals (float)(residual + q4k_quantize_gemv).
 *   residual  device fp32 [M][N], 4-byte aligned; either y itself (an
 *             in-place update of the residual stream) or a buffer that does
 *             not overlap y (a partial overlap returns Q4K_EINVAL).
 * Other arguments, limits and checks as for q4k_quantize_gemv. */
int q4k_quantize_gemv_residual(const void *w, int64_t N, int64_t K, const float *x,
                               int64_t M, const float *residual, float *y, void *stream);

/* One product of a batch for q4k_quantize_gemv_batch (and, with Q6_K
 * weights, q6k_gemv_batch and q6k_quantize_gemv_batch). */
typedef struct q4k_gemv_problem {
    const void *w;     /* device Q4_K weights, N rows x (K/256)*144 bytes, 16-byte aligned */
    const float *x;    /* device fp32 activations [M][K], 16-byte aligned                */
    float *y;          /* device fp32 output [M][N]                                      */
    int64_t N;         /* rows of this matrix, >= 1                                      */
} q4k_gemv_problem;

/* Several independent quantize-and-GEMV products with the same K and M in one
 * launch (e.g. the q, k and v projections of a decode step, or gate and up):
 * for every problem i, y_i = Q8(x_i) * W_i^T, each bit-identical to
 * q4k_quantize_gemv on that problem alone.  `problems` is a host array of
 * `count` entries (1 <= count <= 8), read during the call.  The products must
 * not write overlapping outputs.  Limits and checks as for q4k_quantize_gemv,
 * applied to every problem. */
int q4k_quantize_gemv_batch(const q4k_gemv_problem *problems, int count, int64_t K,
                            int64_t M, void *stream);

/* Prefill GEMM: y[M][N] = Q8(x)[M][K] * W^T for any M >= 1 (the batched
 * prefill over all prompt tokens of "genie-ai-runtime ...", section 3, Path B,
 * whose tensor-core kernel is Path E).  Compute-bound: Q4_K tiles are staged
 * through LDS and converted to integer-valued fp16 operands (sc*q and the Q8
 * codes, both exact), the matrix cores form sc * (each 32-element integer
 * dot) exactly, and the fp32 vector units apply the activation block scale
 * and d; the min term runs on bf16 matrix cores with its fp32 factors split
 * into three exact parts.
 *   workspace        NULL (with workspace_bytes 0), or a device buffer of at
 *                    least q4k_gemm_workspace_bytes() bytes, 256-byte aligned.
 *                    With a workspace, tiles may be split along K across
 *                    workgroups to fill the GPU: a split tile's parts are
 *                    added in a fixed order by the last workgroup to finish,
 *                    so the result bits do not depend on scheduling, and are
 *                    the same with or without a workspace up to fp32 rounding
 *                    of that one sum.  The first 65536 bytes of the workspace
 *                    hold counters that must be zero before the first call
 *                    that uses it (e.g. hipMemset once after allocation);
 *                    every call leaves them zero.  The rest holds partial
 *                    tiles.  Calls sharing a workspace must not overlap.
 * Up to 8 rows (M <= 8, where the rows fit q4k_quantize_gemv's LDS limit)
 * would leave the matrix-core tiles mostly idle: such calls run q4k_gemv's
 * kernels on the prepared rows instead (no workspace used), with q4k_gemv's
 * result bit for bit.
 * Results are deterministic: the same inputs give the same bits on every call.
 * Other arguments and the result contract as for q4k_gemv, without the
 * M <= 8 limit. */
int q4k_gemm(const void *w, int64_t N, int64_t K, const int8_t *codes,
             const float *scales, const int32_t *sums, int64_t M, float *y,
             void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes q4k_gemm and q4k_gemm_batch can use (a constant of the
 * library: 65536 bytes of counters plus 2 * 256 partial tiles of 128 x 128
 * fp32). */
size_t q4k_gemm_workspace_bytes(void);

/* One product of a batch for q4k_gemm_batch. */
typedef struct q4k_gemm_problem {
    const void *w;     /* device Q4_K weights, N rows x (K/256)*144 bytes, 16-byte aligned */
    float *y;          /* device fp32 output [M][N], 4-byte aligned                      */
    int64_t N;         /* rows of this matrix, >= 1                                      */
} q4k_gemm_problem;

/* Several prefill GEMMs against the same Q8 activations in one launch (e.g.
 * the q, k and v projections of a layer, or gate and up): for every problem
 * i, y_i = Q8(x)[M][K] * W_i^T, the same arithmetic as q4k_gemm on that
 * problem alone.  Launching them together fills the GPU where each alone
 * would not; with M <= 8 (the verification rows of drafted tokens, "genie-ai-
 * runtime ...", section 9) all products go out as one launch of one of
 * q4k_gemv's kernels (the matrix-core GEMV where the launch's rows favour it,
 * else the streaming one; either gives q4k_gemv's bits).  `problems` is a host
 * array of `count` entries (1 <= count <= 8),
 * read during the call; outputs must not overlap.  Workspace as for q4k_gemm.
 * Limits and checks as for q4k_gemm, applied to every problem. */
int q4k_gemm_batch(const q4k_gemm_problem *problems, int count, int64_t K,
                   const int8_t *codes, const float *scales, const int32_t *sums,
                   int64_t M, void *workspace, size_t workspace_bytes, void *stream);

/* q4k_gemm_batch without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory or take a caller buffer:
 * code under HIP graph capture, serving loops that forbid allocation on the
 * hot path, harnesses that disallow hipMalloc.  The split-tile counters and
 * partial tiles live in a static device array of the library (33 619 968
 * bytes: 65 536 bytes of counters plus 2 * 256 partial tiles of 128 x 128
 * fp32), one copy per GPU, held from the library's first use on that GPU
 * until the process ends.  Its device address is resolved on the first call
 * on each device.  Every call first clears the counters with a small kernel
 * on `stream` (no memset), then runs the same kernel as q4k_gemm_batch with
 * that array as the workspace, so results equal q4k_gemm_batch with a
 * workspace bit for bit.  No size is refused for want of scratch: a launch
 * whose split-tile counters would not fit runs with whole tiles.  All calls
 * on one GPU share the array: calls that overlap in time on that GPU (on
 * different streams) race and give wrong results.  Returns Q4K_EHIP if the
 * array's address cannot be resolved.  Arguments, limits and checks as for
 * q4k_gemm_batch. */
int q4k_gemm_batch_noalloc(const q4k_gemm_problem *problems, int count, int64_t K,
                           const int8_t *codes, const float *scales, const int32_t *sums,
                           int64_t M, void *stream);

/* Routed-expert grouped GEMV.  n_experts Q4_K matrices of N rows x K columns
 * at expert_stride_bytes from each other (stride >= N*(K/256)*144, multiple of
 * 16).  For token t < T and slot s < topk the expert is ids[t*topk+s].
 * Pairs are grouped by expert on the device (deterministically, in ascending
 * pair order, inside the GEMV kernel), so each touched expert's weights are
 * read once per call however many tokens chose it.  One kernel is enqueued;
 * with routing weights the last workgroup to finish each block of output rows
 * also forms the slot-ordered weighted sum of that block.
 *   ids          device int32 [T][topk], expected in [0, n_experts).  They live
 *                on the device and are not checked on the host; a pair whose id
 *                is out of range is skipped on the device (its per-slot output
 *                row is zero and it adds nothing to a weighted sum).
 *   route_w      NULL: y is per slot, fp32 [T*topk][N];
 *                else device fp32 [T][topk]: y[t] = sum_s route_w[t][s] *
 *                (slot product), summed in slot order 0..topk-1, fp32 [T][N].
 *   act_per_slot 0: activation row t serves every slot of token t (codes
 *                [T][K]); 1: slot (t, s) has its own row t*topk+s (codes
 *                [T*topk][K]).
 *   codes/scales/sums as for q4k_gemv.
 *   workspace    device buffer of at least q4k_moe_workspace_bytes(T, topk,
 *                n_experts, N) bytes, 256-byte aligned.  It starts with
 *                counters (4 bytes per 16 rows of N, rounded up to 256 bytes)
 *                that must be zero before the first call that uses it (e.g.
 *                hipMemset of the whole buffer once after allocation); every
 *                call leaves them zero.  The rest holds the per-slot products
 *                when route_w is given.  Calls sharing a workspace must not
 *                overlap.
 * Limits: 1 <= topk <= n_experts <= 4096, T >= 1, T*topk <= 4096. */
int q4k_moe_gemv(const void *w_experts, int64_t n_experts,
                 int64_t expert_stride_bytes, int64_t N, int64_t K,
                 const int32_t *ids, const float *route_w, int64_t T,
                 int64_t topk, const int8_t *codes, const float *scales,
                 const int32_t *sums, int act_per_slot, float *y,
                 void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes q4k_moe_gemv needs for these sizes (0 on invalid sizes). */
size_t q4k_moe_workspace_bytes(int64_t T, int64_t topk, int64_t n_experts, int64_t N);

/* Routed-expert FFN layer (gate, up, SwiGLU, down, routed sum): for each
 * token t,
 *   y[t] = sum_s route_w[t][s] * Wd[e] . Q8(h),  h = silu(Wg[e] . Q8(x_t)) * (Wu[e] . Q8(x_t)),
 * e = ids[t][s], silu(g) = g / (1 + e^-g) in fp64 rounded to fp32 once.  The
 * result is bit-identical to the unfused chain q4k_quantize_act(x);
 * q4k_moe_gemv(gate), (up); q4k_quantize_act(u, gate = g);
 * q4k_moe_gemv(down, route_w, act_per_slot = 1).  The gate and up products
 * share one launch, and the down launch forms the routed sum itself; for
 * T <= 2 the activations are quantized (and h formed) inside the GEMV
 * kernels, two launches in all (for F <= 1024 the gate|up launch writes
 * Q8(h)); for F <= 1024 and up to 256 pairs each down workgroup sums the
 * slots of its rows itself, with the same bits; for larger T, where that
 * would repeat the
 * work in every workgroup reading a row, the quantizer runs once per row as
 * its own launch (four in all).
 *   w_gate, w_up  n_experts Q4_K matrices of F rows x H columns each, at
 *                 stride_gate_up bytes (>= F*(H/256)*144, multiple of 16)
 *   w_down        n_experts Q4_K matrices of H rows x F columns, at stride_down
 *   ids, route_w  device int32 / fp32 [T][topk]; ids as for q4k_moe_gemv
 *                 (out-of-range ids are skipped); route_w is required
 *   x             device fp32 [T][H], 16-byte aligned; y: device fp32 [T][H]
 *   workspace     device buffer of at least q4k_moe_ffn_workspace_bytes(T,
 *                 topk, n_experts, H, F) bytes, 256-byte aligned: counters of
 *                 the down launch (4 bytes per 16 rows of H, rounded up to 256
 *                 bytes; zero before the first call that uses the buffer, left
 *                 zero by every call), then g, u, the per-slot down products,
 *                 Q8 rows of x and h and the pair grouping; calls sharing a
 *                 workspace must not overlap.
 * Limits as for q4k_moe_gemv; H and F multiples of 256. */
int q4k_moe_ffn(const void *w_gate, const void *w_up, const void *w_down, int64_t n_experts,
                int64_t stride_gate_up, int64_t stride_down, int64_t H, int64_t F,
                const int32_t *ids, const float *route_w, int64_t T, int64_t topk,
                const float *x, float *y, void *workspace, size_t workspace_bytes,
                void *stream);

/* Workspace bytes q4k_moe_ffn needs for these sizes (0 on invalid sizes). */
size_t q4k_moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t n_experts, int64_t H,
                                   int64_t F);

/* Q6_K decode / small-batch GEMV: y[M][N] = Q8(x)[M][K] * W^T for M = 1..8
 * with W in Q6_K, the format real Q4_K_M files keep some tensors in (and the
 * target of the decode kernels of "genie-ai-runtime ...", section 6, "The
 * negatives I kept", Path G):
 * per 256 weights of a row 210 bytes -- ql[128] (low 4 bits of each 6-bit
 * quant q), qh[64] (high 2 bits), int8 sc[16] (one per 16 weights), fp16 d
 * (public GGUF layout) -- and w = d*sc[e/16]*(q[e] - 32).
 *   w       device Q6_K bytes, N rows x (K/256)*210 bytes, 16-byte aligned.
 *   N >= 1, K % 256 == 0, 256 <= K <= 12288, 1 <= M <= 8, and the staged Q8
 *           rows fit one workgroup's LDS: (K/256)*M*416 + 2048*M bytes at most
 *           the device's LDS per workgroup (163840 on MI355X: any K up to
 *           11264 at M = 8, e.g. the 9728-wide down projection).
 *   codes   device int8 [M][K] (16-byte aligned); scales fp32 [M][K/32]
 *           (4-byte aligned) -- as written by q4k_quantize_act (its block
 *           sums are not needed).
 *   y       device fp32 [M][N].
 * fp32 result within a relative error of 2e-3 (absolute 1e-4 near zero) of
 * the exact sum. */
int q6k_gemv(const void *w, int64_t N, int64_t K, const int8_t *codes,
             const float *scales, int64_t M, float *y, void *stream);

/* Q6_K quantize-and-GEMV in one launch: y[M][N] = Q8(x)[M][K] * W^T for fp32
 * activations x (device, [M][K], 16-byte aligned), each workgroup quantizing
 * its Q8 blocks with q4k_quantize_act's arithmetic, so the result equals
 * q4k_quantize_act followed by q6k_gemv bit for bit.  Other arguments and
 * limits as for q6k_gemv. */
int q6k_quantize_gemv(const void *w, int64_t N, int64_t K, const float *x, int64_t M,
                      float *y, void *stream);

/* Several Q6_K GEMVs with the same K and M on the same prepared Q8 rows in
 * one launch (the launch groups of a decode step, e.g. q|k|v or gate|up, on a
 * model whose tensors are Q6_K): for every problem i, y_i = Q8(x)[M][K] *
 * W_i^T, each bit-identical to q6k_gemv on that problem alone.  `problems` is
 * a host array of `count` entries (1 <= count <= 8), read during the call:
 * w the problem's Q6_K weights (N rows x (K/256)*210 bytes, 16-byte aligned),
 * y its output [M][N]; x is not read.  codes and scales as for q6k_gemv.
 * Outputs must not overlap.  Limits and checks as for q6k_gemv, applied to
 * every problem. */
int q6k_gemv_batch(const q4k_gemv_problem *problems, int count, int64_t K, const int8_t *codes,
                   const float *scales, int64_t M, void *stream);

/* q6k_quantize_gemv for several problems with the same K and M in one launch,
 * each with its own fp32 rows x_i [M][K] (16-byte aligned), each output
 * bit-identical to q6k_quantize_gemv on that problem alone.  `problems` as
 * for q6k_gemv_batch, x read; other arguments, limits and checks as for
 * q6k_quantize_gemv, applied to every problem. */
int q6k_quantize_gemv_batch(const q4k_gemv_problem *problems, int count, int64_t K, int64_t M,
                            void *stream);

/* Q6_K prefill GEMM: y[M][N] = Q8(x)[M][K] * W^T with W in Q6_K (layout and
 * weights as for q6k_gemv), the batched product of prefill ("genie-ai-runtime
 * ...", section 3, Path B and Path E) on the Q6_K tensors of a Q4_K_M model
 * (section 6, "The negatives I kept", Path G).  The same tiles, work split and
 * workspace as q4k_gemm: the weights of a 16-weight sub-block enter the fp16
 * matrix cores as two exact integer parts, 16*sc*(q_hi - 2) and sc*q_lo (q =
 * 16 q_hi + q_lo), against the Q8 codes, so each 32-element block's sum of
 * sc*(q - 32)*code is formed in fp32 (exactly while its partial sums stay
 * below 2^24, i.e. for all but near-maximal scales and codes throughout a
 * block); the block scale a and d are applied in fp32.  No sums are needed.
 *   w        device Q6_K bytes, N rows x (K/256)*210 bytes, 16-byte aligned
 *   codes    device int8 [M][K] (16-byte aligned); scales fp32 [M][K/32]
 *   workspace, determinism: as for q4k_gemm.  Any M >= 1, N >= 1,
 *   K % 256 == 0.  fp32 result within a relative error of 2e-3 (absolute
 *   1e-4 near zero) of the exact sum. */
int q6k_gemm(const void *w, int64_t N, int64_t K, const int8_t *codes, const float *scales,
             int64_t M, float *y, void *workspace, size_t workspace_bytes, void *stream);

/* INT8 KV cache (genie-ai-runtime's Path I, section 4 "Memory-first: making
 * every byte count": one absmax scale per (layer, position, kv-head)).  One
 * layer's cache is four device buffers, head-major so that the positions of a
 * kv head are one contiguous stream:
 *   k_codes, v_codes   int8 [n_kv][cap][head_dim]   (16-byte aligned)
 *   k_scales, v_scales fp32 [n_kv][cap]             (4-byte aligned)
 * Entry (h, t) is the vector x of head_dim values of position t and kv head h:
 * scale = fl32(max|x| / 127), code = clamp(round-half-even(fl32(x / scale)),
 * -127, 127); an all-zero vector has scale 0 and codes 0.  The value read back
 * is scale * code.  head_dim is 128 (the only size built).
 *
 * q4k_kv_store: quantize M new positions into the cache:
 *   k, v     device fp32 [M][n_kv][head_dim] (the k and v projection outputs
 *            of M tokens, already position-encoded), 8-byte aligned.
 *   entries (h, pos0 + m) for m < M, h < n_kv are written, nothing else.
 *   1 <= M <= 4096, 1 <= n_kv <= 64, 0 <= pos0, pos0 + M <= cap <= 2^24.
 * Codes and scales are exact (bit for bit the IEEE ones). */
int q4k_kv_store(const float *k, const float *v, int64_t M, int64_t n_kv, int64_t head_dim,
                 int64_t pos0, int64_t cap, int8_t *k_codes, float *k_scales,
                 int8_t *v_codes, float *v_scales, void *stream);

/* Workspace bytes q4k_attn_decode needs for M query tokens and n_head query
 * heads over n_kv kv heads (independent of the context length). */
size_t q4k_attn_workspace_bytes(int64_t M, int64_t n_head, int64_t n_kv);

/* Decode attention over one layer's INT8 cache: M query tokens, the last M
 * positions of a context of n_ctx (token m sits at position n_ctx - M + m and
 * sees positions t < n_ctx - (M - 1 - m)); query head h reads kv head
 * h / (n_head / n_kv) (grouped heads).  For each token m and head h:
 *   s_t = scale * sum_i q[m][h][i] * k_scales[g][t] * k_codes[g][t][i],
 *   p = softmax(s) over the visible t,
 *   out[m][h][i] = sum_t p_t * v_scales[g][t] * v_codes[g][t][i].
 *   q, out     device fp32 [M][n_head][head_dim], 16-byte aligned.
 *   1 <= M <= 8, n_head % n_kv == 0, n_head / n_kv <= 8, n_kv <= 64,
 *   M <= n_ctx <= cap <= 2^24, head_dim == 128.
 *   workspace  device buffer of at least q4k_attn_workspace_bytes(M, n_head,
 *              n_kv) bytes, 256-byte aligned; its first 4096 bytes are
 *              counters that must be zero before the first call that uses it
 *              (e.g. hipMemset once after allocation); every call leaves them
 *              zero.  Calls sharing a workspace must not overlap.
 * One kernel is enqueued.  The context is split into chunks across
 * workgroups; the chunk partials are merged in chunk order, so the result bits
 * do not depend on scheduling.  fp32 result within a relative error of 2e-3
 * (absolute 1e-4 near zero) of the exact value of the formula above. */
int q4k_attn_decode(const float *q, int64_t M, int64_t n_head, int64_t n_kv, int64_t head_dim,
                    const int8_t *k_codes, const float *k_scales, const int8_t *v_codes,
                    const float *v_scales, int64_t cap, int64_t n_ctx, float scale, float *out,
                    void *workspace, size_t workspace_bytes, void *stream);

/* Measurement aids, not on the product path: the practical ceilings that
 * bench.py reports beside the decode launches.
 * q4k_ceiling_stream_read: `grid` workgroups of 256 threads read `bytes`
 *   (multiple of 16) of the device buffer `buf` (16-byte aligned) in 16-byte
 *   loads, grid-stride, and write one word per workgroup to `sink` (device,
 *   >= grid words): the bytes of a launch moved with no arithmetic.
 * q4k_ceiling_empty: `grid` workgroups of an empty kernel: the cost of a
 *   kernel boundary alone.
 * q4k_ceiling_mfma_valu: `grid` workgroups of 8 waves.  With bit 0 of `what`
 *   set, waves 0-3 (one per SIMD) issue `iters` x 4 v_mfma_f32_32x32x16_f16
 *   in four independent accumulator chains; with bit 1 set, waves 4-7 (one
 *   per SIMD, beside them) issue `iters` x `vrep` x 32 fp32 fmas in sixteen
 *   independent chains.  Timing what = 1, 2 and 3 shows how far the two
 *   kinds of work overlap on one SIMD -- the question that bounds the prefill
 *   GEMM, whose fp32 epilogue follows its matrix-core ops.  One float per
 *   workgroup goes to `sink` (device, >= grid floats).  1 <= iters <= 2^24,
 *   0 <= vrep <= 64, 1 <= what <= 3.
 * 1 <= grid <= 2^20. */
int q4k_ceiling_stream_read(const void *buf, int64_t bytes, int64_t grid, unsigned *sink,
                            void *stream);
int q4k_ceiling_empty(int64_t grid, void *stream);
int q4k_ceiling_mfma_valu(int64_t grid, int64_t iters, int vrep, int what, float *sink,
                          void *stream);

/* Static description of a status code. */
const char *q4k_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* Q4K_H */
