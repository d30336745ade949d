// Routed-expert grouped GEMV (the mixture-of-experts layers of "I'm making LLMs
// work on small and old devices": intro, expert pager; each token touches only
// its selected experts, so the bytes read per token are those experts').
//
// Three launches on the caller's stream:
//  1. group_kernel (one workgroup): from ids[T][topk] build, per expert, the
//     count and offset of its (token, slot) pairs and the pair list in
//     ascending pair order, plus the ascending list of touched experts.
//     Counts use LDS atomics (order-free), offsets a one-wave scan, and each
//     pair's slot is its rank among earlier pairs of the same expert, so the
//     tables are deterministic.  A pair whose id is outside [0, n_experts)
//     belongs to no expert: it is skipped (its per-slot output row is zero).
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
constexpr int kChunk = 4;            // activation rows per pass over a weight tile
constexpr int kRowTiles = 2;         // 8-row tiles per workgroup

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

// Exclusive prefix sum of v over one wave (64 lanes); returns the lane's
// exclusive prefix and the wave total in *total.
__device__ __forceinline__ int wave_exclusive_scan(int v, int *total) {
    const int lane = threadIdx.x & 63;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    *total = __shfl(x, 63, 64);
    return x - v;
}

__global__ __launch_bounds__(1024) void group_kernel(const int32_t *__restrict__ ids, int P,
                                                     int E, int *__restrict__ counts,
                                                     int *__restrict__ offsets,
                                                     int *__restrict__ act,
                                                     int *__restrict__ nact,
                                                     int *__restrict__ pairs,
                                                     float *__restrict__ y_zero_rows, int N) {
    __shared__ int s_ids[kMoeMaxPairs];
    __shared__ int s_cnt[kMoeMaxExperts];
    __shared__ int s_off[kMoeMaxExperts];
    const int tid = threadIdx.x, nt = blockDim.x;
    for (int e = tid; e < E; e += nt) s_cnt[e] = 0;
    __syncthreads();
    // Counts: LDS atomics (the count does not depend on their order).
    for (int p = tid; p < P; p += nt) {
        const int e = ids[p];
        s_ids[p] = e;
        if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
    }
    __syncthreads();
    // Offsets and the touched-expert list: the first wave scans E in chunks
    // of 64 experts.
    if (tid < 64) {
        int base = 0, abase = 0;
        for (int e0 = 0; e0 < E; e0 += 64) {
            const int e = e0 + tid;
            const int c = e < E ? s_cnt[e] : 0;
            int tot, atot;
            const int ex = wave_exclusive_scan(c, &tot);
            const int aex = wave_exclusive_scan(c > 0 ? 1 : 0, &atot);
            if (e < E) {
                s_off[e] = base + ex;
                offsets[e] = base + ex;
                counts[e] = c;
                if (c > 0) act[abase + aex] = e;
            }
            base += tot;
            abase += atot;
        }
        if (tid == 0) {
            offsets[E] = base;
            *nact = abase;
        }
    }
    __syncthreads();
    // Placement in ascending pair order: the rank of pair p within its expert
    // is the number of earlier pairs with the same id.
    for (int p = tid; p < P; p += nt) {
        const int e = s_ids[p];
        if (e < 0 || e >= E) continue;
        int r = 0;
        for (int q = 0; q < p; ++q) r += (s_ids[q] == e);
        pairs[s_off[e] + r] = p;
    }
    // Per-slot output without routing weights: rows of skipped pairs are zero.
    if (y_zero_rows) {
        for (int p = 0; p < P; ++p) {
            const int e = s_ids[p];
            if (e >= 0 && e < E) continue;
            for (int n = tid; n < N; n += nt) y_zero_rows[(int64_t)p * N + n] = 0.0f;
        }
    }
}

// One workgroup: touched expert act[blockIdx.y], rows [16*blockIdx.x, +16)
// (two 8-row tiles), all of that expert's pairs in chunks of kChunk
// activation rows.  Same lane mapping and load discipline as the decode GEMV:
// activation loads first, then the weight loads of the wave's column, all
// branch-free from clamped addresses; a wave takes further columns in later
// passes when K has more than 16 super-blocks.
__global__ __launch_bounds__(1024) void moe_gemv_kernel(
    const uint8_t *__restrict__ w, int64_t stride, int N, int nsb, int topk,
    int act_per_slot, const int8_t *__restrict__ codes, const float *__restrict__ scales,
    const int32_t *__restrict__ sums, const int *__restrict__ counts,
    const int *__restrict__ offsets, const int *__restrict__ act, const int *__restrict__ nact,
    const int *__restrict__ pairs, float *__restrict__ out) {
    constexpr int R = 8 * kRowTiles;
    __shared__ float red[kMaxWaves][R][kChunk];
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
    int row[kRowTiles];
#pragma unroll
    for (int t = 0; t < kRowTiles; ++t)   // rows past N: computed, never written
        row[t] = min((int)blockIdx.x * R + 8 * t + grp, N - 1);

    for (int c0 = 0; c0 < cnt; c0 += kChunk) {
        const int mc = min(kChunk, cnt - c0);
        int arow[kChunk];
#pragma unroll
        for (int m = 0; m < kChunk; ++m) {
            const int p = pairs[off + c0 + min(m, mc - 1)];
            arow[m] = act_per_slot ? p : p / topk;
        }
        float acc[kRowTiles][kChunk];
#pragma unroll
        for (int t = 0; t < kRowTiles; ++t)
#pragma unroll
            for (int m = 0; m < kChunk; ++m) acc[t][m] = 0.0f;
        for (int b = wave; b < nsb; b += nwaves) {
            i32x4 cA[kChunk], cB[kChunk];
            float a[kChunk];
            int s[kChunk];
#pragma unroll
            for (int m = 0; m < kChunk; ++m) {
                const int8_t *cm = codes + (int64_t)arow[m] * K + 256 * b;
                cA[m] = *reinterpret_cast<const i32x4 *>(cm + L.offA);
                cB[m] = *reinterpret_cast<const i32x4 *>(cm + L.offB);
                a[m] = scales[(int64_t)arow[m] * nblk + 8 * b + L.l];
                s[m] = sums[(int64_t)arow[m] * nblk + 8 * b + L.l];
            }
            __builtin_amdgcn_sched_barrier(0);
            u32x4 hd[kRowTiles], qw[kRowTiles];
#pragma unroll
            for (int t = 0; t < kRowTiles; ++t) {
                const uint8_t *sb = we + (int64_t)row[t] * row_bytes + (int64_t)b * 144;
                hd[t] = load_stream16(sb);
                qw[t] = load_stream16(sb + 16 + 16 * L.l);
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < kRowTiles; ++t) {
                float ds, dm;
                decode_scale(L, hd[t], ds, dm);
                int qlo[4], qhi[4];
                unpack_nibbles(qw[t], qlo, qhi);
#pragma unroll
                for (int m = 0; m < kChunk; ++m) {
                    if (m < mc) {   // wave-uniform
                        const int D = subblock_dot(L, qlo, qhi, cA[m], cB[m]);
                        acc[t][m] = fmaf(a[m], fmaf(ds, (float)D, -(dm * (float)s[m])), acc[t][m]);
                    }
                }
            }
        }
#pragma unroll
        for (int t = 0; t < kRowTiles; ++t)
#pragma unroll
            for (int m = 0; m < kChunk; ++m) {
                const float v = group8_sum(acc[t][m]);
                if (L.l == 0) red[wave][8 * t + grp][m] = v;
            }
        __syncthreads();
        for (int i = threadIdx.x; i < R * kChunk; i += blockDim.x) {
            const int r = i / kChunk, m = i % kChunk;
            const int n = (int)blockIdx.x * R + r;
            if (m < mc && n < N) {
                float v = 0.0f;
                for (int wv = 0; wv < nwaves; ++wv) v += red[wv][r][m];
                out[(int64_t)pairs[off + c0 + m] * N + n] = v;
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
                       counts, offsets, act, nact, pairs, route_w ? nullptr : y, (int)N);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const int nsb = (int)(K / kQK);
    const int max_active = (int)(P < n_experts ? P : n_experts);
    dim3 grid((unsigned)((N + 8 * kRowTiles - 1) / (8 * kRowTiles)), (unsigned)max_active);
    float *dst = route_w ? z : y;
    // One column per wave and pass; a wave takes further columns in later
    // passes when K has more than 16 super-blocks.
    const int nw = nsb < kMaxWaves ? nsb : kMaxWaves;
    hipLaunchKernelGGL(moe_gemv_kernel, grid, dim3(64 * nw), 0, stream, w, stride, (int)N,
                       nsb, (int)topk, act_per_slot, codes, scales, sums, counts, offsets, act,
                       nact, pairs, dst);
    err = hipGetLastError();
    if (err != hipSuccess || !route_w) return err;

    const int64_t total = T * N;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, z, route_w, ids, (int)n_experts, (int)T, (int)topk, (int)N, y);
    return hipGetLastError();
}

}  // namespace q4k
