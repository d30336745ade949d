// Routed-expert grouped GEMV (the mixture-of-experts layers of "I'm making LLMs
// work on small and old devices": intro, expert pager; each token touches only
// its selected experts, so the bytes read per token are those experts').
//
// One launch (two with routing weights) on the caller's stream:
//  1. moe_gemv_kernel: grid = row blocks x touched-expert slots (+ one row of
//     workgroups that zero the per-slot rows of skipped pairs).  Every
//     workgroup groups the pairs itself from ids[T][topk] (at most 4096 ids,
//     in LDS): slot a is the a-th smallest touched expert, and its pairs are
//     taken in ascending pair order -- deterministic, no tables in memory and
//     no separate grouping launch.  It then computes one block of that
//     expert's rows for all of its pairs (the decode GEMV's lane layout,
//     every load in flight before the arithmetic), MC pairs per pass with the
//     weights in registers, so every touched expert's weights are streamed
//     from HBM once per call (again from L2 for each further MC).  A pair
//     whose id is outside [0, n_experts) belongs to no expert: it is skipped
//     (its per-slot output row is zero).
//  2. reduce_kernel (only with routing weights): y[t] = sum over slots s in
//     order 0..topk-1 of route_w[t][s] * z[t*topk+s] -- fixed order, no float
//     atomics, bit-reproducible.
#include <algorithm>

#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kMoeWaves = 4;         // waves per workgroup, at most
constexpr int kMoeV = 8;             // row groups per lane
constexpr int kMoeMC = 4;            // pairs per pass over a weight block

// Workspace: the per-slot products z [T*topk][N] when routing weights are given.
size_t ws_bytes(int64_t T, int64_t topk, int64_t N) {
    return (size_t)((4 * T * topk * N + 255) & ~int64_t(255));
}

// Dynamic LDS of moe_gemv_kernel: ids (padded to 4), expert flags, pair list.
size_t moe_lds_bytes(int P, int E) { return sizeof(int) * ((size_t)((P + 3) & ~3) + (size_t)E + P); }

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

// One workgroup: the touched expert of slot blockIdx.y and a block of RB = RG*V
// of its rows; all of that expert's pairs, MC at a time.  Lane layout as in
// the decode GEMV (stream_gemv.h): 8 lanes per 144-byte super-block, a wave's
// 8 lane groups are RG rows x S = 8/RG column slots, a lane holds V row
// groups; W waves x S slots cover W*S super-block columns per pass (more
// passes when K is wider).  Per pass a wave issues the activation loads of
// its column for the chunk's pairs and then every weight load of its V row
// groups before any arithmetic, so the block is in flight at once.  Per lane
// the terms of a (row, pair) add up over the passes; the 8 lanes of a group
// (DPP), then the W waves and their S slots (LDS, in a fixed order) complete
// a row: a fixed order for a given (N, K).
// With zero_skipped, the last row of workgroups (blockIdx.y == gridDim.y - 1)
// writes zeros to the rows of pairs whose id is out of range instead.
template <int V, int MC>
__global__ __launch_bounds__(256) void moe_gemv_kernel(
    const uint8_t *__restrict__ w, int64_t stride, int N, int nsb, int lg_rg, int topk,
    int act_per_slot, const int8_t *__restrict__ codes, const float *__restrict__ scales,
    const int32_t *__restrict__ sums, const int32_t *__restrict__ ids, int P, int E,
    int zero_skipped, float *__restrict__ out) {
    extern __shared__ __attribute__((aligned(16))) int lds_m[];
    int *s_ids = lds_m;                      // [P rounded up to 4]
    int *s_flag = s_ids + ((P + 3) & ~3);    // [E] expert touched
    int *s_pairs = s_flag + E;               // [P] this slot's pairs, ascending
    __shared__ float red[kMoeWaves][8 * V][MC];
    __shared__ int s_wt[kMoeWaves];
    __shared__ int s_e;
    const int RG = 1 << lg_rg, S = 8 >> lg_rg, RB = RG * V;
    const int row_base = (int)blockIdx.x * RB;
    if (row_base >= N) return;                     // uniform per workgroup
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nw = nt >> 6;

    // ---- grouping, in LDS: ids, touched-expert flags
    for (int p = tid; p < P; p += nt) s_ids[p] = ids[p];
    for (int e = tid; e < E; e += nt) s_flag[e] = 0;
    if (tid == 0) s_e = -1;
    __syncthreads();
    for (int p = tid; p < P; p += nt) {
        const int e = s_ids[p];
        if (e >= 0 && e < E) s_flag[e] = 1;        // same value from every writer
    }
    __syncthreads();
    if (zero_skipped && (int)blockIdx.y == (int)gridDim.y - 1) {
        // per-slot rows of skipped pairs are zero (this block of rows)
        for (int p = 0; p < P; ++p) {
            const int e = s_ids[p];
            if (e >= 0 && e < E) continue;
            for (int n = row_base + tid; n < min(N, row_base + RB); n += nt)
                out[(int64_t)p * N + n] = 0.0f;
        }
        return;
    }
    // slot a = blockIdx.y is the a-th smallest touched expert: each thread
    // counts the flags of a range of experts, a block scan places the ranges
    {
        const int a = (int)blockIdx.y;
        const int per = (E + nt - 1) / nt;
        const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
        int c = 0;
        for (int e = e0; e < e1; ++e) c += s_flag[e];
        int wtot;
        const int ex = wave_exclusive_scan(c, &wtot);
        if (lane == 0) s_wt[wave] = wtot;
        __syncthreads();
        int base = ex;
        for (int k = 0; k < wave; ++k) base += s_wt[k];
        if (a >= base && a < base + c) {
            int k = a - base;
            for (int e = e0; e < e1; ++e)
                if (s_flag[e] && k-- == 0) {
                    s_e = e;
                    break;
                }
        }
        __syncthreads();
    }
    const int e = s_e;
    if (e < 0) return;                             // uniform: slot past the touched experts
    // the expert's pairs in ascending order: per round of nt pairs, wave
    // ballots and the earlier waves' counts place each one
    int cnt = 0;
    for (int p0 = 0; p0 < P; p0 += nt) {
        const int p = p0 + tid;
        const bool f = p < P && s_ids[p] == e;
        const unsigned long long mask = __ballot(f);
        const int below = __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                                    __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0));
        __syncthreads();                           // s_wt free again
        if (lane == 0) s_wt[wave] = __popcll(mask);
        __syncthreads();
        int base = cnt;
        for (int k = 0; k < wave; ++k) base += s_wt[k];
        if (f) s_pairs[base + below] = p;
        for (int k = 0; k < nw; ++k) cnt += s_wt[k];
    }
    __syncthreads();

    const int g = lane >> 3, r = g & (RG - 1), sl = g >> lg_rg;
    const LaneMap L(lane & 7);
    const ScaleBits SB(lane & 7);
    const int K = nsb * 256, nblk = nsb * 8;
    const unsigned row_bytes = (unsigned)nsb * 144u;
    // the block's first row in 64 bits, 32-bit offsets within it
    const uint8_t *__restrict__ wb = w + (int64_t)e * stride + (int64_t)row_base * row_bytes;
    const int span = nw * S;                       // columns per pass
    const int npass = (nsb + span - 1) / span;

    for (int c0 = 0; c0 < cnt; c0 += MC) {
        const int mc = min(MC, cnt - c0);
        int arow[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int pr = s_pairs[c0 + min(m, mc - 1)];
            arow[m] = act_per_slot ? pr : pr / topk;
        }
        float acc[V][MC];
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int m = 0; m < MC; ++m) acc[v][m] = 0.0f;
        for (int pass = 0; pass < npass; ++pass) {
            const int b = (pass * nw + wave) * S + sl;
            const bool live = b < nsb;                 // per lane group
            const int bc = min(b, nsb - 1);
            i32x4 cA[MC], cB[MC];
            float a[MC], sm[MC];
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const int8_t *cm = codes + (int64_t)arow[m] * K + 256 * bc;
                cA[m] = *reinterpret_cast<const i32x4 *>(cm + L.offA);
                cB[m] = *reinterpret_cast<const i32x4 *>(cm + L.offB);
                a[m] = scales[(int64_t)arow[m] * nblk + 8 * bc + L.l];
                sm[m] = (float)sums[(int64_t)arow[m] * nblk + 8 * bc + L.l];
            }
            __builtin_amdgcn_sched_barrier(0);
            // branch-free weight loads: rows past N read row N-1 (never written);
            // the header as one dword per lane, spread over the lane quad at use
            unsigned hd[V];
            u32x4 qw[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const unsigned rr = (unsigned)(min(row_base + v * RG + r, N - 1) - row_base);
                const unsigned o = rr * row_bytes + (unsigned)bc * 144u;
                hd[v] = __builtin_nontemporal_load(
                    reinterpret_cast<const unsigned *>(wb + (o + 4u * (lane & 3))));
                qw[v] = load_stream16(wb + (o + 16u + 16u * L.l));
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float ds, dm;
                decode_scale_bits(SB, quad_gather(hd[v]), ds, dm);
                int qlo[4], qhi[4];
                unpack_nibbles(qw[v], qlo, qhi);
#pragma unroll
                for (int m = 0; m < MC; ++m) {
                    if (m < mc) {   // wave-uniform
                        const int D = subblock_dot(L, qlo, qhi, cA[m], cB[m]);
                        const float t = a[m] * fmaf(ds, (float)D, -(dm * sm[m]));
                        acc[v][m] += live ? t : 0.0f;
                    }
                }
            }
        }
        // a row's terms: the 8 lanes of a group (DPP), then over the waves and
        // each wave's S slots (LDS, wave-major order)
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const float t = group8_sum(acc[v][m]);
                if (L.l == 0) red[wave][sl * RB + v * RG + r][m] = t;
            }
        __syncthreads();
        for (int i = threadIdx.x; i < RB * MC; i += blockDim.x) {
            const int rr = i / MC, m = i % MC;
            const int n = row_base + rr;
            if (m < mc && n < N) {
                float t = 0.0f;
                for (int wv = 0; wv < nw; ++wv)
                    for (int k = 0; k < S; ++k) t += red[wv][k * RB + rr][m];
                out[(int64_t)s_pairs[c0 + m] * N + n] = t;
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
    (void)n_experts;
    return ws_bytes(T, topk, N);
}

hipError_t launch_moe_gemv(const uint8_t *w, int64_t n_experts, int64_t stride, int64_t N,
                           int64_t K, const int32_t *ids, const float *route_w, int64_t T,
                           int64_t topk, const int8_t *codes, const float *scales,
                           const int32_t *sums, int act_per_slot, float *y, void *workspace,
                           hipStream_t stream) {
    float *z = static_cast<float *>(workspace);
    const int P = (int)(T * topk);
    const int E = (int)n_experts;
    const int slots = P < E ? P : E;
    const int nsb = (int)(K / kQK);
    // Column slots per wave: enough that at most kMoeWaves waves cover K in
    // one pass (S = 8 at most; wider K takes several passes).
    int lg_rg = 3;
    while (lg_rg > 0 && (nsb + (8 >> lg_rg) - 1) / (8 >> lg_rg) > kMoeWaves) --lg_rg;
    const int S = 8 >> lg_rg;
    const int nw = std::min(kMoeWaves, (nsb + S - 1) / S);
    const int RB = (1 << lg_rg) * kMoeV;
    const int zero_skipped = route_w ? 0 : 1;
    dim3 grid((unsigned)((N + RB - 1) / RB), (unsigned)(slots + zero_skipped));
    float *dst = route_w ? z : y;
    const size_t lds = moe_lds_bytes(P, E);
    // Pairs per pass: an expert has at most T pairs when each token lists
    // distinct experts, so small T needs no wider pass (more pairs only take
    // more passes).
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(64 * nw), lds, stream, w, stride, (int)N, nsb, lg_rg,
                           (int)topk, act_per_slot, codes, scales, sums, ids, P, E, zero_skipped,
                           dst);
    };
    if (T == 1)
        go(moe_gemv_kernel<kMoeV, 1>);
    else if (T == 2)
        go(moe_gemv_kernel<kMoeV, 2>);
    else
        go(moe_gemv_kernel<kMoeV, kMoeMC>);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || !route_w) return err;

    const int64_t total = T * N;
    hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                       stream, z, route_w, ids, (int)n_experts, (int)T, (int)topk, (int)N, y);
    return hipGetLastError();
}

}  // namespace q4k
