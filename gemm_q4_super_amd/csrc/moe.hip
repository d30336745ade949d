// Routed-expert grouped GEMV (the mixture-of-experts layers of "I'm making LLMs
// work on small and old devices": intro, expert pager; each token touches only
// its selected experts, so the bytes read per token are those experts').
//
// Three launches on the caller's stream:
//  1. group_kernel (one workgroup): from ids[T][topk] build, per expert, the
//     count and offset of its (token, slot) pairs and the pair list in
//     ascending pair order, plus the ascending list of touched experts.  One
//     thread per expert scans the ids, so the result is deterministic and
//     needs no atomics.  A pair whose id is outside [0, n_experts) belongs to
//     no expert: it is skipped (its per-slot output row is written as zeros).
//  2. moe_gemv_kernel: grid = row tiles x touched-expert slots.  Each workgroup
//     takes one touched expert and one tile of its rows, and computes that
//     tile for all of the expert's pairs (in chunks of 8 activation rows), so
//     every touched expert's weights are streamed from HBM once per call.
//  3. reduce_kernel (only with routing weights): y[t] = sum over slots s in
//     order 0..topk-1 of route_w[t][s] * z[t*topk+s] -- fixed order, no float
//     atomics, bit-reproducible.
#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kChunk = 8;            // activation rows per pass over a weight tile

struct WsLayout {
    int64_t counts, offsets, act, nact, pairs, z;   // byte offsets
    size_t bytes;
};

int64_t align256(int64_t v) { return (v + 255) & ~int64_t(255); }

WsLayout layout(int64_t T, int64_t topk, int64_t E, int64_t N) {
    WsLayout L;
    const int64_t P = T * topk;
    L.counts = 0;
    L.offsets = align256(L.counts + 4 * E);
    L.act = align256(L.offsets + 4 * (E + 1));
    L.nact = align256(L.act + 4 * E);
    L.pairs = align256(L.nact + 4);
    L.z = align256(L.pairs + 4 * P);
    L.bytes = (size_t)align256(L.z + 4 * P * N);
    return L;
}

__global__ __launch_bounds__(1024) void group_kernel(const int32_t *__restrict__ ids, int P,
                                                     int E, int topk, int *__restrict__ counts,
                                                     int *__restrict__ offsets,
                                                     int *__restrict__ act,
                                                     int *__restrict__ nact,
                                                     int *__restrict__ pairs,
                                                     float *__restrict__ y_zero_rows, int N) {
    __shared__ int s_ids[kMoeMaxPairs];
    __shared__ int s_cnt[kMoeMaxExperts];
    __shared__ int s_flag[kMoeMaxExperts];
    const int tid = threadIdx.x;
    for (int p = tid; p < P; p += blockDim.x) s_ids[p] = ids[p];
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        int c = 0;
        for (int p = 0; p < P; ++p) c += (s_ids[p] == e);
        s_cnt[e] = c;
        s_flag[e] = c > 0;
    }
    __syncthreads();
    if (tid == 0) {
        // Exclusive scans (E is at most a few thousand; one pass).
        int off = 0, na = 0;
        for (int e = 0; e < E; ++e) {
            offsets[e] = off;
            counts[e] = s_cnt[e];
            off += s_cnt[e];
            if (s_flag[e]) act[na++] = e;
            s_flag[e] = off - s_cnt[e];   // reuse: start offset of expert e
        }
        offsets[E] = off;
        *nact = na;
    }
    __syncthreads();
    for (int e = tid; e < E; e += blockDim.x) {
        if (s_cnt[e] == 0) continue;
        int k = s_flag[e];
        for (int p = 0; p < P; ++p)
            if (s_ids[p] == e) pairs[k++] = p;
    }
    // Per-slot output without routing weights: rows of skipped pairs are zero.
    if (y_zero_rows) {
        for (int p = 0; p < P; ++p) {
            const int e = s_ids[p];
            if (e >= 0 && e < E) continue;
            for (int n = tid; n < N; n += blockDim.x) y_zero_rows[(int64_t)p * N + n] = 0.0f;
        }
    }
    (void)topk;
}

// One workgroup: expert act[blockIdx.y], rows [8*blockIdx.x, +8), all pairs.
__global__ __launch_bounds__(1024) void moe_gemv_kernel(
    const uint8_t *__restrict__ w, int64_t stride, int N, int nsb, int cpw, int topk,
    int act_per_slot, const int8_t *__restrict__ codes, const float *__restrict__ scales,
    const int32_t *__restrict__ sums, const int *__restrict__ counts,
    const int *__restrict__ offsets, const int *__restrict__ act, const int *__restrict__ nact,
    const int *__restrict__ pairs, float *__restrict__ out) {
    __shared__ float red[kMaxWaves][8][kChunk];
    if ((int)blockIdx.y >= *nact) return;          // uniform per workgroup
    const int e = act[blockIdx.y];
    const int cnt = counts[e], off = offsets[e];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int grp = lane >> 3;
    const LaneMap L(lane & 7);
    const int K = nsb * 256, nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * 144;
    const uint8_t *we = w + (int64_t)e * stride;
    const int row = blockIdx.x * 8 + grp;
    const int b_begin = wave * cpw, b_end = min(nsb, b_begin + cpw);

    for (int c0 = 0; c0 < cnt; c0 += kChunk) {
        const int mc = min(kChunk, cnt - c0);
        int arow[kChunk];
#pragma unroll
        for (int m = 0; m < kChunk; ++m) {
            const int p = pairs[off + c0 + min(m, mc - 1)];
            arow[m] = act_per_slot ? p : p / topk;
        }
        float acc[kChunk];
#pragma unroll
        for (int m = 0; m < kChunk; ++m) acc[m] = 0.0f;
        for (int b = b_begin; b < b_end; ++b) {
            u32x4 hd = (u32x4){0u, 0u, 0u, 0u}, qw = (u32x4){0u, 0u, 0u, 0u};
            if (row < N) {
                const uint8_t *sb = we + (int64_t)row * row_bytes + (int64_t)b * 144;
                hd = load_stream16(sb);
                qw = load_stream16(sb + 16 + 16 * L.l);
            }
            float ds, dm;
            decode_scale(L, hd, ds, dm);
            int qlo[4], qhi[4];
            unpack_nibbles(qw, qlo, qhi);
#pragma unroll
            for (int m = 0; m < kChunk; ++m) {
                if (m < mc) {   // wave-uniform
                    const int8_t *cm = codes + (int64_t)arow[m] * K + 256 * b;
                    const i32x4 cA = *reinterpret_cast<const i32x4 *>(cm + L.offA);
                    const i32x4 cB = *reinterpret_cast<const i32x4 *>(cm + L.offB);
                    const float a = scales[(int64_t)arow[m] * nblk + 8 * b + L.l];
                    const float s = (float)sums[(int64_t)arow[m] * nblk + 8 * b + L.l];
                    const int D = subblock_dot(L, qlo, qhi, cA, cB);
                    acc[m] = fmaf(a, ds * (float)D - dm * s, acc[m]);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < kChunk; ++m) {
            const float v = group8_sum(acc[m]);
            if (L.l == 0) red[wave][grp][m] = v;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < 8 * kChunk; i += blockDim.x) {
            const int r = i / kChunk, m = i % kChunk;
            if (m < mc && blockIdx.x * 8 + r < N) {
                float v = 0.0f;
                for (int wv = 0; wv < nwaves; ++wv) v += red[wv][r][m];
                out[(int64_t)pairs[off + c0 + m] * N + blockIdx.x * 8 + r] = v;
            }
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(256) void reduce_kernel(const float *__restrict__ z,
                                                     const float *__restrict__ route_w,
                                                     const int32_t *__restrict__ ids, int E,
                                                     int T, int topk, int N,
                                                     float *__restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)T * N) return;
    const int t = (int)(i / N), n = (int)(i % N);
    float v = 0.0f;
    for (int s = 0; s < topk; ++s) {
        const int p = t * topk + s;
        const int e = ids[p];
        if (e >= 0 && e < E) v = fmaf(route_w[p], z[(int64_t)p * N + n], v);
    }
    y[i] = v;
}

}  // namespace

size_t moe_workspace_bytes(int64_t T, int64_t topk, int64_t n_experts, int64_t N) {
    return layout(T, topk, n_experts, N).bytes;
}

hipError_t launch_moe_gemv(const uint8_t *w, int64_t n_experts, int64_t stride, int64_t N,
                           int64_t K, const int32_t *ids, const float *route_w, int64_t T,
                           int64_t topk, const int8_t *codes, const float *scales,
                           const int32_t *sums, int act_per_slot, float *y, void *workspace,
                           hipStream_t stream) {
    const WsLayout Lo = layout(T, topk, n_experts, N);
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    int *counts = reinterpret_cast<int *>(ws + Lo.counts);
    int *offsets = reinterpret_cast<int *>(ws + Lo.offsets);
    int *act = reinterpret_cast<int *>(ws + Lo.act);
    int *nact = reinterpret_cast<int *>(ws + Lo.nact);
    int *pairs = reinterpret_cast<int *>(ws + Lo.pairs);
    float *z = reinterpret_cast<float *>(ws + Lo.z);
    const int P = (int)(T * topk);

    hipLaunchKernelGGL(group_kernel, dim3(1), dim3(1024), 0, stream, ids, P, (int)n_experts,
                       (int)topk, counts, offsets, act, nact, pairs, route_w ? nullptr : y,
                       (int)N);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const int nsb = (int)(K / kQK);
    const int cpw = (nsb + kMaxWaves - 1) / kMaxWaves;
    const int nwaves = (nsb + cpw - 1) / cpw;
    const int max_active = (int)(P < n_experts ? P : n_experts);
    dim3 grid((unsigned)((N + 7) / 8), (unsigned)max_active);
    hipLaunchKernelGGL(moe_gemv_kernel, grid, dim3(64 * nwaves), 0, stream, w, stride, (int)N,
                       nsb, cpw, (int)topk, act_per_slot, codes, scales, sums, counts, offsets,
                       act, nact, pairs, route_w ? z : y);
    err = hipGetLastError();
    if (err != hipSuccess || !route_w) return err;

    const int64_t total = T * N;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, z, route_w, ids, (int)n_experts, (int)T, (int)topk, (int)N, y);
    return hipGetLastError();
}

}  // namespace q4k
