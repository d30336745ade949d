// Routed-expert grouped GEMV and expert FFN layer (the mixture-of-experts
// layers of "I'm making LLMs work on small and old devices": intro, expert
// pager; each token touches only its selected experts, so the bytes read per
// token are those experts').
//
// moe_kernel: grid = row blocks x touched-expert slots (x 2 when the gate and
// up projections share a launch; + one row of workgroups that zero the
// per-slot rows of skipped pairs).  Every workgroup groups the pairs itself
// from ids[T][topk] (at most 4096 ids, in LDS): slot a is the a-th smallest
// touched expert, and its pairs are taken in ascending pair order --
// deterministic, no tables in memory and no separate grouping launch (the
// routed-expert layer above two tokens instead reads a table that its
// quantizer launch makes once, moe_quantize_group_kernel).  It then
// computes one block of that expert's rows for all of its pairs (the decode
// GEMV's lane layout, every load in flight before the arithmetic), MC pairs
// per pass with the weights in registers, so every touched expert's weights
// are streamed from HBM once per call (again from L2 for each further MC).  A
// pair whose id is outside [0, n_experts) belongs to no expert: it is skipped
// (its per-slot output row is zero).  The activation of a pair is
//  * Q8 rows prepared by q4k_quantize_act (q4k_moe_gemv), or
//  * fp32 rows quantized in the kernel (the FFN's gate|up launch), or
//  * SwiGLU(g, u) of fp32 rows, quantized in the kernel (the FFN's down),
// all through the same quantizer and SwiGLU arithmetic as q4k_quantize_act,
// so the fused layer's codes equal the unfused chain's bit for bit.
// With routing weights the same launch also forms y[t] = sum over slots s in
// order 0..topk-1 of route_w[t][s] * z[t*topk+s]: the per-slot products z go
// to the workspace through agent-coherent stores, and the last workgroup to
// finish a row block (a counter per row block) adds them up for that block --
// fixed order, no float atomics, bit-reproducible, no separate launch.
//
// Layers of up to 256 pairs take shorter paths with the same bits: for one or
// two tokens the gate|up launch holds the same rows of both projections in
// each workgroup and writes Q8(SwiGLU(g, u)) itself (ACT_F32_H8), and the
// down launch (moe_down_sum_kernel for one token, moe_down_rows_kernel for
// more) gives each workgroup a few output rows and every pair, summing the
// slots in slot order inside the workgroup -- no per-slot products or
// counters.
#include <algorithm>

#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kMoeWaves = 4;         // waves per workgroup, at most (8 for ACT_F32_H8)
constexpr int kMoeV = 8;             // row groups per lane
constexpr int kMoeMC = 4;            // pairs per pass over a weight block
constexpr int kMoeMC2MaxT = 8;       // up to this many tokens, 2 pairs per pass (fewer
                                     // registers, more workgroups per CU: T = 4 46.1 -> 43.9 us)
constexpr int kStageBytes = 256 + 64;   // one staged column: codes, 8 scales, 8 sums
constexpr int kStageSlots = 2;          // column slots per wave, at most (the staged columns)
constexpr int kFuseMaxT = 2;            // tokens up to which the FFN quantizes in its GEMVs
constexpr int kDownSumSlots = 8;        // slots of a one-token layer whose down launch sums them in
                                        // each workgroup
constexpr int kRowsMaxPairs = 256;      // pairs up to which the down launch takes every pair per
                                        // row block (moe_down_rows_kernel)
constexpr int kRowsChunk = 8;           // experts whose weights a lane holds at once there

// ACT_F32_H8: fp32 rows quantized in the kernel, as ACT_F32, in a launch whose
// workgroups each hold the same rows of both projections (gate in the first
// half of the block, up in the second) and write Q8(SwiGLU(g, u)) of them.
enum { ACT_Q8 = 0, ACT_F32 = 1, ACT_SWIGLU = 2, ACT_F32_H8 = 3 };

struct MoeArgs {
    const uint8_t *w[2];       // expert matrices (w[1]: second projection of a shared launch)
    float *out[2];
    int64_t stride;            // bytes between experts
    int N, nsb, lg_rg, topk, act_per_slot, P, E, slots, zero_skipped;
    const int8_t *codes;       // ACT_Q8
    const float *scales;
    const int32_t *sums;
    const float *xa, *xb;      // ACT_F32: x [.][K]; ACT_SWIGLU: g, u [P][K]
    const int32_t *ids;
    int direct;                // one token: slot a is pair a (no grouping)
    // the grouping made once for the call (moe_quantize_group_kernel), or
    // null: slot a's expert tab_e[a] (-1 past the touched ones) and its pairs
    // tab_p[tab_s[a] .. tab_s[a + 1])
    const int *tab_e, *tab_s, *tab_p;
    // Routed sum inside the launch (null cnt: none): the per-slot products go
    // to out[0] through agent-coherent stores, and the last workgroup of each
    // row block writes y[t][n] = sum over slots s in order of
    // route_w[t][s] * out[0][t*topk+s][n].  cnt: one counter per row block,
    // zero between calls.
    const float *route_w;
    float *y;
    unsigned *cnt;
    int T;
    // ACT_F32_H8: Q8 rows of h = SwiGLU(g, u), one per pair [P][N]
    int8_t *hc;
    float *hs;
    int32_t *hsu;
};

__host__ __device__ constexpr size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

// LDS of the grouping: ids (padded to 4), expert flags, pair list.
__host__ __device__ constexpr size_t group_bytes(int P, int E) {
    return sizeof(int) * ((size_t)((P + 3) & ~3) + (size_t)E + P);
}

// Dynamic LDS of moe_kernel: the grouping and the staged Q8 columns of each
// wave.
size_t moe_lds_bytes(int P, int E, int nw, int S, int MC) {
    return align16(group_bytes(P, E)) + (size_t)nw * S * MC * kStageBytes;
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

// End of a workgroup of a launch with the routed sum inside: once every
// per-slot product the workgroup stored has completed, it counts itself on its
// row block's counter; the last of the row block's gridDim.y workgroups adds
// the slots of every token in slot order (one fma per slot, in order)
// and returns the counter to zero.  Every workgroup of the row block calls
// this exactly once, also those whose slot has no expert.
__device__ void routed_sum(const MoeArgs &A, const int *s_ids, int row_base, int RB) {
    __shared__ unsigned last;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(A.cnt + blockIdx.x, 1u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT) == gridDim.y - 1;
    __syncthreads();
    if (!last) return;
    const int N = A.N, topk = A.topk, E = A.E;
    const int rows = min(RB, N - row_base);
    const int total = A.T * rows;
    // one output per thread when they fit the workgroup, else kOut per
    // thread at a time; the slots are taken kSlotStep at a time with every
    // load of a step issued before its first fma (slots past topk repeat the
    // last slot and are not added: selects, so no load waits behind a branch)
    constexpr int kSlotStep = 8;
    if (total <= (int)blockDim.x) {
        if ((int)threadIdx.x < total) {
            const int t = threadIdx.x / rows, n = row_base + threadIdx.x % rows;
            float v = 0.0f;
            for (int s0 = 0; s0 < topk; s0 += kSlotStep) {
                int ee[kSlotStep];
                float zz[kSlotStep], ww[kSlotStep];
#pragma unroll
                for (int j = 0; j < kSlotStep; ++j) {
                    const int p = t * topk + min(s0 + j, topk - 1);
                    ee[j] = s_ids[p];
                    zz[j] = __hip_atomic_load(A.out[0] + (int64_t)p * N + n, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                    ww[j] = A.route_w[p];
                }
#pragma unroll
                for (int j = 0; j < kSlotStep; ++j)
                    v = s0 + j < topk && ee[j] >= 0 && ee[j] < E ? fmaf(ww[j], zz[j], v) : v;
            }
            A.y[(int64_t)t * N + n] = v;
        }
    }
    constexpr int kOut = 4;
    for (int i0 = threadIdx.x; i0 < total && total > (int)blockDim.x; i0 += kOut * blockDim.x) {
        int t[kOut], n[kOut];
        float v[kOut];
#pragma unroll
        for (int k = 0; k < kOut; ++k) {
            const int i = min(i0 + k * (int)blockDim.x, total - 1);
            t[k] = i / rows;
            n[k] = row_base + i % rows;
            v[k] = 0.0f;
        }
        for (int s0 = 0; s0 < topk; s0 += kSlotStep) {
            int ee[kOut][kSlotStep];
            float zz[kOut][kSlotStep], ww[kOut][kSlotStep];
#pragma unroll
            for (int k = 0; k < kOut; ++k)
#pragma unroll
                for (int j = 0; j < kSlotStep; ++j) {
                    const int p = t[k] * topk + min(s0 + j, topk - 1);
                    ee[k][j] = s_ids[p];
                    zz[k][j] = __hip_atomic_load(A.out[0] + (int64_t)p * N + n[k], __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
                    ww[k][j] = A.route_w[p];
                }
#pragma unroll
            for (int k = 0; k < kOut; ++k)
#pragma unroll
                for (int j = 0; j < kSlotStep; ++j)
                    v[k] = s0 + j < topk && ee[k][j] >= 0 && ee[k][j] < E
                               ? fmaf(ww[k][j], zz[k][j], v[k]) : v[k];
        }
#pragma unroll
        for (int k = 0; k < kOut; ++k)
            if (i0 + k * (int)blockDim.x < total) A.y[(int64_t)t[k] * N + n[k]] = v[k];
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(A.cnt + blockIdx.x, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// One workgroup: the touched expert of slot a (blockIdx.y, past the first
// projection's slots for the second) and a block of RB = RG*V of its rows;
// all of that expert's pairs, MC at a time.  Lane layout as in the decode
// GEMV (stream_gemv.h): 8 lanes per 144-byte super-block, a wave's 8 lane
// groups are RG rows x S = 8/RG column slots, a lane holds V row groups; W
// waves x S slots cover W*S super-block columns per pass (more passes when K
// is wider).  Per pass a wave issues the activation loads of its columns for
// the chunk's pairs and then every weight load of its V row groups before any
// arithmetic, so the block is in flight at once; the activation then goes
// into the wave's own LDS stage (no workgroup barrier): prepared Q8 rows
// copied (four wide loads per pass instead of four loads per pair per lane),
// fp32 rows quantized.  Per lane
// the terms of a (row, pair) add up over the passes; the 8 lanes of a group
// (DPP), then the W waves and their S slots (LDS, in a fixed order) complete a
// row: a fixed order for a given K (the launch shape depends on K alone).
// With zero_skipped, the last row of workgroups (blockIdx.y == gridDim.y - 1)
// writes zeros to the rows of pairs whose id is out of range instead.
template <int V, int MC, int MODE>
__global__ __launch_bounds__(MODE == ACT_F32_H8 ? 512 : 256) void moe_kernel(const MoeArgs A) {
    extern __shared__ __attribute__((aligned(16))) int lds_m[];
    const int P = A.P, E = A.E, N = A.N, nsb = A.nsb, lg_rg = A.lg_rg;
    int *s_ids = lds_m;                      // [P rounded up to 4]
    int *s_flag = s_ids + ((P + 3) & ~3);    // [E] expert touched
    int *s_pairs = s_flag + E;               // [P] this slot's pairs, ascending
    constexpr bool H8 = MODE == ACT_F32_H8;
    constexpr int NWMAX = H8 ? 2 * kMoeWaves : kMoeWaves;
    __shared__ float red[NWMAX][8 * V][MC];
    __shared__ int s_wt[NWMAX];
    __shared__ int s_e;
    static_assert(!H8 || MC == 1, "one pair per workgroup when h is formed");
    __shared__ float hrow[H8 ? 8 * V : 1];         // H8: g then u of the block's rows
    const int RG = 1 << lg_rg, S = 8 >> lg_rg, RB = RG * V;
    const int RBr = H8 ? RB / 2 : RB;              // rows of each projection
    const int row_base = (int)blockIdx.x * RBr;
    if (row_base >= N) return;                     // uniform per workgroup
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int nw = nt >> 6;

    int mi, e, cnt;
    int pair_a = -1;                               // the slot's one pair (direct calls), else -1
    if (A.tab_e) {                                 // uniform: the call's grouping table
        mi = (int)blockIdx.y >= A.slots ? 1 : 0;
        const int a = (int)blockIdx.y - mi * A.slots;
        e = A.tab_e[a];
        if (e < 0) return;                         // slot past the touched experts
        const int q0 = A.tab_s[a];
        cnt = A.tab_s[a + 1] - q0;
        for (int p = tid; p < cnt; p += nt) s_pairs[p] = A.tab_p[q0 + p];
        __syncthreads();
    } else if (A.direct && !A.zero_skipped && !A.cnt) {
        // one pair per slot, nothing else to do per call: the slot's id read
        // by every thread, no staging of the ids and no barrier
        mi = (int)blockIdx.y >= A.slots ? 1 : 0;
        pair_a = (int)blockIdx.y - mi * A.slots;
        e = A.ids[pair_a];
        if (e < 0 || e >= E) return;               // uniform: the pair belongs to no expert
        cnt = 1;
    } else {
        // ---- grouping, in LDS: ids, touched-expert flags (a one-token call maps
        // slot a to pair a directly: no flags, scan or pair list)
        const bool direct = A.direct != 0;             // uniform
        for (int p = tid; p < P; p += nt) s_ids[p] = A.ids[p];
        if (!direct)
            for (int e = tid; e < E; e += nt) s_flag[e] = 0;
        if (tid == 0) s_e = -1;
        __syncthreads();
        if (!direct) {
            for (int p = tid; p < P; p += nt) {
                const int e = s_ids[p];
                if (e >= 0 && e < E) s_flag[e] = 1;    // same value from every writer
            }
            __syncthreads();
        }
        if (A.zero_skipped && (int)blockIdx.y == (int)gridDim.y - 1) {
            // per-slot rows of skipped pairs are zero (this block of rows)
            for (int p = 0; p < P; ++p) {
                const int e = s_ids[p];
                if (e >= 0 && e < E) continue;
                for (int n = row_base + tid; n < min(N, row_base + RBr); n += nt)
                    A.out[0][(int64_t)p * N + n] = 0.0f;
            }
            return;
        }
        mi = (int)blockIdx.y >= A.slots ? 1 : 0;         // which projection
        if (direct) {
            if (tid == 0) {
                const int a = (int)blockIdx.y - mi * A.slots;
                const int ea = s_ids[a];
                s_e = ea >= 0 && ea < E ? ea : -1;
                s_pairs[0] = a;
            }
            __syncthreads();
        } else {
            // slot a is the a-th smallest touched expert: each thread counts the
            // flags of a range of experts, a block scan places the ranges
            const int a = (int)blockIdx.y - mi * A.slots;
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
        e = s_e;
        if (e < 0) {                                   // uniform: slot past the touched experts
            if (A.cnt) routed_sum(A, s_ids, row_base, RB);
            return;
        }
        // the expert's pairs in ascending order: per round of nt pairs, wave
        // ballots and the earlier waves' counts place each one
        cnt = direct ? 1 : 0;
        for (int p0 = 0; p0 < P && !direct; p0 += nt) {
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
    }

    const int g = lane >> 3, r = g & (RG - 1), sl = g >> lg_rg;
    const LaneMap L(lane & 7);
    const ScaleBits SB(lane & 7);
    const int K = nsb * 256, nblk = nsb * 8;
    const unsigned row_bytes = (unsigned)nsb * 144u;
    float *__restrict__ out = A.out[mi];
    // the block's first row in 64 bits, 32-bit offsets within it
    const uint8_t *__restrict__ wb =
        A.w[mi] + (int64_t)e * A.stride + (int64_t)row_base * row_bytes;
    // H8: row groups V/2.. are the same rows of the second projection
    const uint8_t *__restrict__ wb_up =
        H8 ? A.w[1] + (int64_t)e * A.stride + (int64_t)row_base * row_bytes : wb;
    const int span = nw * S;                       // columns per pass
    const int npass = (nsb + span - 1) / span;
    // this wave's activation stage: [S][MC] columns of codes, scales, sums
    uint8_t *stage = reinterpret_cast<uint8_t *>(lds_m) + align16(group_bytes(P, E)) +
                     (size_t)wave * S * MC * kStageBytes;
    const int qblk = lane >> 3, qsub = lane & 7;   // quantizer layout: block, 4 values

    for (int c0 = 0; c0 < cnt; c0 += MC) {
        const int mc = min(MC, cnt - c0);
        int arow[MC];
#pragma unroll
        for (int m = 0; m < MC; ++m) {
            const int pr = pair_a >= 0 ? pair_a : s_pairs[c0 + min(m, mc - 1)];
            arow[m] = A.act_per_slot ? pr : pr / A.topk;
        }
        float acc[V][MC];
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int m = 0; m < MC; ++m) acc[v][m] = 0.0f;
        for (int pass = 0; pass < npass; ++pass) {
            const int wcol = (pass * nw + wave) * S;   // the wave's first column
            const int b = wcol + sl;
            const bool live = b < nsb;                 // per lane group
            const int bc = min(b, nsb - 1);
            i32x4 cA[MC], cB[MC];
            float a[MC], sm[MC];
            // launches use S <= kStageSlots (so RG >= 4): at most 2 MC staged columns
            constexpr int SX = MODE == ACT_Q8 ? 1 : kStageSlots;
            constexpr int SU = MODE == ACT_SWIGLU ? kStageSlots : 1;
            f32x4 xv[SX][MC], xu[SU][MC];
            // prepared Q8 rows: column j of pair m is staged as 16 lanes x 16 bytes
            // of codes (column-pair k = j*MC + m on lanes 16(k%4).., two loads)
            // and 8 lanes x 4 bytes of scales and of sums (lanes 8k..)
            constexpr int QK = MODE == ACT_Q8 ? (kStageSlots * MC + 3) / 4 : 1;
            i32x4 qc[QK];
            float qa = 0.0f;
            int qs = 0;
            if constexpr (MODE == ACT_Q8) {
                auto row_of = [&](int mm) {   // arow[mm] for a per-lane mm (from LDS)
                    const int pr = pair_a >= 0 ? pair_a : s_pairs[c0 + min(mm, mc - 1)];
                    return A.act_per_slot ? pr : pr / A.topk;
                };
#pragma unroll
                for (int i = 0; i < QK; ++i) {
                    const int k = min((lane >> 4) + 4 * i, S * MC - 1);
                    const int col = min(wcol + k / MC, nsb - 1);
                    qc[i] = *reinterpret_cast<const i32x4 *>(
                        A.codes + (int64_t)row_of(k % MC) * K + 256 * col + 16 * (lane & 15));
                }
                const int k = min(lane >> 3, S * MC - 1);
                const int col = min(wcol + k / MC, nsb - 1);
                const int64_t so = (int64_t)row_of(k % MC) * nblk + 8 * col + (lane & 7);
                qa = A.scales[so];
                qs = A.sums[so];
            } else {
                // fp32 activation of the wave's S columns, quantizer layout
#pragma unroll
                for (int j = 0; j < SX; ++j) {
                    if (j >= S) break;                 // wave-uniform
                    const int col = min(wcol + j, nsb - 1);
#pragma unroll
                    for (int m = 0; m < MC; ++m) {
                        const int64_t o = (int64_t)arow[m] * K + 256 * col + 32 * qblk + 4 * qsub;
                        xv[j][m] = *reinterpret_cast<const f32x4 *>(A.xa + o);
                        if constexpr (MODE == ACT_SWIGLU)
                            xu[j][m] = *reinterpret_cast<const f32x4 *>(A.xb + o);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            // branch-free weight loads: rows past N read row N-1 (never written);
            // the header as one dword per lane, spread over the lane quad at use
            unsigned hd[V];
            u32x4 qw[V];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const bool up = H8 && v >= V / 2;      // compile-time per v
                const int vv = up ? v - V / 2 : v;
                const uint8_t *__restrict__ wv = up ? wb_up : wb;
                const unsigned rr = (unsigned)(min(row_base + vv * RG + r, N - 1) - row_base);
                const unsigned o = rr * row_bytes + (unsigned)bc * 144u;
                hd[v] = *reinterpret_cast<const unsigned *>(wv + (o + 4u * (lane & 3)));
                qw[v] = load_weights16(wv + (o + 16u + 16u * L.l));
            }
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (MODE == ACT_Q8) {
                // copy the prepared rows into the wave's stage
#pragma unroll
                for (int i = 0; i < QK; ++i) {
                    const int k = (lane >> 4) + 4 * i;
                    if (k < S * MC)
                        *reinterpret_cast<i32x4 *>(stage + (size_t)k * kStageBytes +
                                                   16 * (lane & 15)) = qc[i];
                }
                if ((lane >> 3) < S * MC) {
                    uint8_t *st = stage + (size_t)(lane >> 3) * kStageBytes;
                    reinterpret_cast<float *>(st + 256)[lane & 7] = qa;
                    reinterpret_cast<float *>(st + 288)[lane & 7] = (float)qs;
                }
            } else {
                // quantize into the wave's stage
#pragma unroll
                for (int j = 0; j < SX; ++j) {
                    if (j >= S) break;
#pragma unroll
                    for (int m = 0; m < MC; ++m) {
                        f32x4 v4 = xv[j][m];
                        if constexpr (MODE == ACT_SWIGLU) v4 = swiglu4(v4, xu[j][m]);
                        const Q8Lane q = quantize_block8(v4);
                        uint8_t *st = stage + (size_t)(j * MC + m) * kStageBytes;
                        *reinterpret_cast<unsigned *>(st + 32 * qblk + 4 * qsub) = q.codes;
                        if (qsub == 0) {
                            reinterpret_cast<float *>(st + 256)[qblk] = q.d;
                            reinterpret_cast<float *>(st + 288)[qblk] = (float)q.sum;
                        }
                    }
                }
            }
            // read the stage in the dot layout
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the stage is written
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int m = 0; m < MC; ++m) {
                const uint8_t *st = stage + (size_t)(sl * MC + m) * kStageBytes;
                cA[m] = *reinterpret_cast<const i32x4 *>(st + L.offA);
                cB[m] = *reinterpret_cast<const i32x4 *>(st + L.offB);
                a[m] = reinterpret_cast<const float *>(st + 256)[L.l];
                sm[m] = reinterpret_cast<const float *>(st + 288)[L.l];
            }
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
            // the stage is rewritten by the next pass: reads done first
            __builtin_amdgcn_s_waitcnt(0xc07f);
            __builtin_amdgcn_wave_barrier();
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
            const int n = row_base + (H8 ? rr % RBr : rr);
            if (m < mc && n < N) {
                float t = 0.0f;
                if (S == 1) {                          // uniform
                    // every wave's term requested before the first add (rows of
                    // waves past nw are read and not added)
                    float tw[NWMAX];
#pragma unroll
                    for (int wv = 0; wv < NWMAX; ++wv) tw[wv] = red[wv][rr][m];
#pragma unroll
                    for (int wv = 0; wv < NWMAX; ++wv) t = wv < nw ? t + tw[wv] : t;
                } else {
                    for (int wv = 0; wv < nw; ++wv)
                        for (int k = 0; k < S; ++k) t += red[wv][k * RB + rr][m];
                }
                if constexpr (H8) {
                    hrow[rr] = t;
                } else {
                    float *o = out + (int64_t)(pair_a >= 0 ? pair_a : s_pairs[c0 + m]) * N + n;
                    if (A.cnt)
                        __hip_atomic_store(o, t, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    else
                        *o = t;
                }
            }
        }
        __syncthreads();
        if constexpr (H8) {
            // h = SwiGLU(g, u) of the block's rows, quantized in blocks of 32
            // (8 lanes x 4 values each, the quantizer's own layout): the same
            // codes the down launch would form from g and u
            if (wave == 0) {
                // one value per lane (the fp64 exp is the long part), then the
                // quantizer's 8 lanes x 4 values per block
                for (int j = lane; j < RBr; j += 64) hrow[j] = swiglu1(hrow[j], hrow[RBr + j]);
                __builtin_amdgcn_s_waitcnt(0xc07f);
                __builtin_amdgcn_wave_barrier();
                const int nb = RBr / 32;
                const int bq = min(lane >> 3, nb - 1), q4 = lane & 7;
                const int j = 32 * bq + 4 * q4;
                const f32x4 h4 = {hrow[j], hrow[j + 1], hrow[j + 2], hrow[j + 3]};
                const Q8Lane q = quantize_block8(h4);
                if ((lane >> 3) < nb) {
                    const int pr = pair_a >= 0 ? pair_a : s_pairs[c0];
                    *reinterpret_cast<unsigned *>(A.hc + (int64_t)pr * N + row_base + j) = q.codes;
                    if (q4 == 0) {
                        const int64_t so = (int64_t)pr * (N / 32) + row_base / 32 + bq;
                        A.hs[so] = q.d;
                        A.hsu[so] = q.sum;
                    }
                }
            }
            __syncthreads();
        }
    }
    if (A.cnt) routed_sum(A, s_ids, row_base, RB);
}

// Down projection of a one-token layer with the routed sum in the workgroup:
// a workgroup takes RG = 8 rows of the output and every slot of the token
// (each slot's expert weights for those rows), so no workgroup waits for
// another.  Its waves are nwc column waves (one column of a pass each) times
// PM/PH slot sets of PH slots (the slots' weights in registers at once).  The
// lane layout, the staging of the prepared Q8 rows of h and the order of every
// sum are those of moe_kernel for the same K (S = 1: K <= 1024): a slot's
// product z is the same float, and y[n] = sum over slots s in order of
// route_w[s] * z[s][n] (slots whose id is out of range skipped) the same as
// the last workgroup of a row block forms it there.
template <int PM, int PH>
__global__ __launch_bounds__(512) void moe_down_sum_kernel(const MoeArgs A) {
    static_assert(PM % PH == 0 && PH % 4 == 0 && PH <= 8, "slot sets of 4 or 8");
    constexpr int kSets = PM / PH;
    __shared__ float red[kMoeWaves][8][PM];
    __shared__ __attribute__((aligned(16))) uint8_t stage[kMoeWaves * kSets][PH][kStageBytes];
    const int P = A.P, E = A.E, N = A.N, nsb = A.nsb;
    const int row_base = (int)blockIdx.x * 8;
    if (row_base >= N) return;                     // uniform per workgroup
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nwc = ((int)blockDim.x >> 6) / kSets;  // column waves
    const int set = wave / nwc, wc = wave % nwc;
    const int p0 = set * PH;                       // the wave's first slot
    const int r = lane >> 3;                       // row of the lane group
    const LaneMap L(lane & 7);
    const ScaleBits SB(lane & 7);
    const int K = nsb * 256, nblk = nsb * 8;
    const unsigned row_bytes = (unsigned)nsb * 144u;
    const unsigned rr = (unsigned)min(row_base + r, N - 1);
    // the slots' experts (scalar loads); an out-of-range id reads expert 0 and
    // is left out of the sum; slots past P repeat slot P-1's addresses (cache
    // hits) and are left out too
    int ex[PH];
#pragma unroll
    for (int p = 0; p < PH; ++p) {
        const int e = A.ids[min(p0 + p, P - 1)];
        ex[p] = e >= 0 && e < E ? e : 0;
    }
    // every slot's id and routing weight for the final sum, requested now
    // rather than after the barrier (slots past P repeat slot P-1 and are
    // not added)
    int eid[PM];
    float rw[PM];
#pragma unroll
    for (int p = 0; p < PM; ++p) {
        eid[p] = A.ids[min(p, P - 1)];
        rw[p] = A.route_w[min(p, P - 1)];
    }
    float acc[PH];
#pragma unroll
    for (int p = 0; p < PH; ++p) acc[p] = 0.0f;
    const int npass = (nsb + nwc - 1) / nwc;
    for (int pass = 0; pass < npass; ++pass) {
        const int b = pass * nwc + wc;             // the wave's column
        const bool live = b < nsb;
        const int bc = min(b, nsb - 1);
        // prepared Q8 rows of the slots: codes as 16 lanes x 16 bytes per slot
        // (slots p0 + 4i + lane/16), scales and sums as 8 lanes x 4 bytes
        // (slot p0 + lane/8)
        i32x4 qc[PH / 4];
#pragma unroll
        for (int i = 0; i < PH / 4; ++i) {
            const int k = min(p0 + (lane >> 4) + 4 * i, P - 1);
            qc[i] = *reinterpret_cast<const i32x4 *>(A.codes + (int64_t)k * K + 256 * bc +
                                                     16 * (lane & 15));
        }
        const int ks = min(p0 + (lane >> 3), P - 1);
        const int64_t so = (int64_t)ks * nblk + 8 * bc + (lane & 7);
        const float qa = A.scales[so];
        const int qs = A.sums[so];
        __builtin_amdgcn_sched_barrier(0);
        unsigned hd[PH];
        u32x4 qw[PH];
#pragma unroll
        for (int p = 0; p < PH; ++p) {
            const uint8_t *__restrict__ wp = A.w[0] + (int64_t)ex[p] * A.stride;
            const int64_t o = (int64_t)rr * row_bytes + (int64_t)bc * 144;
            hd[p] = *reinterpret_cast<const unsigned *>(wp + o + 4 * (lane & 3));
            qw[p] = load_weights16(wp + o + 16 + 16 * L.l);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < PH / 4; ++i)
            *reinterpret_cast<i32x4 *>(&stage[wave][(lane >> 4) + 4 * i][16 * (lane & 15)]) = qc[i];
        if ((lane >> 3) < PH) {
            reinterpret_cast<float *>(&stage[wave][lane >> 3][256])[lane & 7] = qa;
            reinterpret_cast<float *>(&stage[wave][lane >> 3][288])[lane & 7] = (float)qs;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0): the stage is written
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int p = 0; p < PH; ++p) {
            float ds, dm;
            decode_scale_bits(SB, quad_gather(hd[p]), ds, dm);
            const uint8_t *st = &stage[wave][p][0];
            const i32x4 cA = *reinterpret_cast<const i32x4 *>(st + L.offA);
            const i32x4 cB = *reinterpret_cast<const i32x4 *>(st + L.offB);
            const float a = reinterpret_cast<const float *>(st + 256)[L.l];
            const float sm = reinterpret_cast<const float *>(st + 288)[L.l];
            int qlo[4], qhi[4];
            unpack_nibbles(qw[p], qlo, qhi);
            const int D = subblock_dot(L, qlo, qhi, cA, cB);
            const float t = a * fmaf(ds, (float)D, -(dm * sm));
            acc[p] += live ? t : 0.0f;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);       // the next pass rewrites the stage
        __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int p = 0; p < PH; ++p) {
        const float t = group8_sum(acc[p]);
        if (L.l == 0) red[wc][r][p0 + p] = t;
    }
    __syncthreads();
    if (tid < 8 && row_base + tid < N) {
        // every slot's column terms requested before the first add; terms of
        // waves past nwc and slots past P are read and not added (selects, so
        // no read waits behind a branch)
        float zr[PM][kMoeWaves];
#pragma unroll
        for (int p = 0; p < PM; ++p)
#pragma unroll
            for (int c = 0; c < kMoeWaves; ++c) zr[p][c] = red[c][tid][p];
        float v = 0.0f;
#pragma unroll
        for (int p = 0; p < PM; ++p) {
            float z = 0.0f;
#pragma unroll
            for (int c = 0; c < kMoeWaves; ++c) z = c < nwc ? z + zr[p][c] : z;
            v = p < P && eid[p] >= 0 && eid[p] < E ? fmaf(rw[p], z, v) : v;
        }
        A.y[row_base + tid] = v;
    }
}

// Down projection with the routed sum in the workgroup, for several tokens
// (P <= kRowsMaxPairs pairs, K <= 1024 so that a pass is one column per
// wave): a workgroup takes RG = 8 output rows, sorts the valid pairs by
// expert once (a count per expert, a scan, cursors), and takes them XB at a
// time: each pair's expert weights for the wave's column of the 8 rows and
// its prepared Q8 row of h, all requested together, then the dots.  Its waves
// are nwc column waves times sets of them that take alternate chunks, so
// several chunks' loads are in flight.  The per-pair products stay in LDS and
// the routed sum is formed from them in slot order: no per-slot products in
// memory, no counters.  Lane layout and the order of every sum are those of
// moe_kernel for the same K, so the bits equal the chain's.
template <int XB>
__global__ __launch_bounds__(1024) void moe_down_rows_kernel(const MoeArgs A) {
    extern __shared__ __attribute__((aligned(16))) int lds_r[];
    __shared__ int s_wt[16];
    __shared__ int s_tot[1];
    const int P = A.P, E = A.E, N = A.N, nsb = A.nsb, topk = A.topk;
    const int row_base = (int)blockIdx.x * 8;
    if (row_base >= N) return;                     // uniform per workgroup
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    const int nwc = nsb;                           // column waves (one pass)
    const int sets = (nt >> 6) / nwc, set = wave / nwc, wc = wave % nwc;
    int *s_ids = lds_r;                            // [P rounded up to 4]
    int *cnt = s_ids + ((P + 3) & ~3);             // [E] pairs per expert, then cursor
    int *sorted = cnt + E;                         // [P] valid pairs by expert
    float *s_rw = reinterpret_cast<float *>(sorted + P);   // [P] routing weights
    float *red = reinterpret_cast<float *>(
        reinterpret_cast<uint8_t *>(lds_r) + align16(sizeof(int) * (((P + 3) & ~3) + (size_t)E + 2 * P)));
    uint8_t *stage = reinterpret_cast<uint8_t *>(red) + align16(sizeof(float) * (size_t)nwc * 8 * P) +
                     (size_t)wave * XB * kStageBytes;

    // ---- grouping: a count per expert, a scan of the counts over expert
    // ranges, then each valid pair placed at its expert's cursor
    for (int p = tid; p < P; p += nt) {
        s_ids[p] = A.ids[p];
        s_rw[p] = A.route_w[p];                    // for the routed sum at the end
    }
    for (int e = tid; e < E; e += nt) cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += nt) {
        const int e = s_ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    {
        const int per = (E + nt - 1) / nt;
        const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
        int c = 0;
        for (int e = e0; e < e1; ++e) c += cnt[e];
        int wtot;
        const int ex = wave_exclusive_scan(c, &wtot);
        if (lane == 0) s_wt[wave] = wtot;
        __syncthreads();
        int bc = ex;
        for (int k = 0; k < wave; ++k) bc += s_wt[k];
        for (int e = e0; e < e1; ++e) {
            const int n = cnt[e];
            cnt[e] = bc;                           // cursor of the expert's pairs
            bc += n;
        }
        if (tid == nt - 1) s_tot[0] = bc;          // valid pairs
    }
    __syncthreads();
    for (int p = tid; p < P; p += nt) {
        const int e = s_ids[p];
        if (e >= 0 && e < E) sorted[atomicAdd(&cnt[e], 1)] = p;   // order within an expert is free
    }
    __syncthreads();

    const int r = lane >> 3;                       // row of the lane group
    const LaneMap L(lane & 7);
    const ScaleBits SB(lane & 7);
    const int K = nsb * 256, nblk = nsb * 8;
    const unsigned row_bytes = (unsigned)nsb * 144u;
    // the lane's row and column within an expert's matrix
    const unsigned lo = (unsigned)min(row_base + r, N - 1) * row_bytes + (unsigned)wc * 144u;
    // Chunks of XB consecutive pairs in expert order, every load of a chunk
    // issued together: each pair's expert rows (pairs of one expert sit side
    // by side, so the repeats hit in cache), then its Q8 rows of h for the
    // wave's column -- one wait per chunk, and the wave sets' chunks in
    // flight side by side.
    const int nv = s_tot[0];
    const int nchunks = (nv + XB - 1) / XB;
    static_assert(XB == 8, "two code loads and one scale load per lane");
    for (int c = set; c < nchunks; c += sets) {
        const int q0 = c * XB;
        unsigned hd[XB];
        u32x4 qw[XB];
#pragma unroll
        for (int k = 0; k < XB; ++k) {
            const int e = s_ids[sorted[min(q0 + k, nv - 1)]];
            const uint8_t *__restrict__ wp = A.w[0] + (int64_t)e * A.stride;
            hd[k] = *reinterpret_cast<const unsigned *>(wp + (lo + 4u * (lane & 3)));
            qw[k] = load_weights16(wp + (lo + 16u + 16u * L.l));
        }
        // codes as 16 lanes x 16 bytes per pair (pairs 4i + lane/16), scales
        // and sums as 8 lanes x 4 bytes (pair lane/8)
        i32x4 cv[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int pc = sorted[min(q0 + (lane >> 4) + 4 * i, nv - 1)];
            cv[i] = *reinterpret_cast<const i32x4 *>(A.codes + (int64_t)pc * K + 256 * wc + 16 * (lane & 15));
        }
        const int ps = sorted[min(q0 + (lane >> 3), nv - 1)];
        const int64_t so = (int64_t)ps * nblk + 8 * wc + (lane & 7);
        const float qa = A.scales[so];
        const int qs = A.sums[so];
#pragma unroll
        for (int i = 0; i < 2; ++i)
            *reinterpret_cast<i32x4 *>(stage + (size_t)((lane >> 4) + 4 * i) * kStageBytes + 16 * (lane & 15)) = cv[i];
        reinterpret_cast<float *>(stage + (size_t)(lane >> 3) * kStageBytes + 256)[lane & 7] = qa;
        reinterpret_cast<float *>(stage + (size_t)(lane >> 3) * kStageBytes + 288)[lane & 7] = (float)qs;
        __builtin_amdgcn_s_waitcnt(0xc07f);       // lgkmcnt(0): the stage is written
        __builtin_amdgcn_wave_barrier();
        const int nq = min(XB, nv - q0);
#pragma unroll
        for (int k = 0; k < XB; ++k) {
            if (k >= nq) break;                    // uniform
            float ds, dm;
            decode_scale_bits(SB, quad_gather(hd[k]), ds, dm);
            int qlo[4], qhi[4];
            unpack_nibbles(qw[k], qlo, qhi);
            const uint8_t *sj = stage + (size_t)k * kStageBytes;
            const i32x4 cA = *reinterpret_cast<const i32x4 *>(sj + L.offA);
            const i32x4 cB = *reinterpret_cast<const i32x4 *>(sj + L.offB);
            const float a = reinterpret_cast<const float *>(sj + 256)[L.l];
            const float sm = reinterpret_cast<const float *>(sj + 288)[L.l];
            const int D = subblock_dot(L, qlo, qhi, cA, cB);
            float acc = 0.0f;
            acc += a * fmaf(ds, (float)D, -(dm * sm));
            const float t = group8_sum(acc);
            if (L.l == 0) red[((size_t)wc * 8 + r) * P + sorted[q0 + k]] = t;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);       // the stage is rewritten next
        __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    // y[t][n] = sum over slots s in order of route_w * z, z the column terms in order
    const int T = P / topk;
    for (int i = tid; i < T * 8; i += nt) {
        const int t = i >> 3, rw = i & 7, n = row_base + rw;
        if (n >= N) continue;
        float v = 0.0f;
        // 8 slots at a time, every read of them requested before the first add
        // (slots past topk repeat the last slot and column waves past nwc the
        // last wave; neither is added)
        for (int s0 = 0; s0 < topk; s0 += 8) {
            int ee[8];
            float ww[8], zr[8][kMoeWaves];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int p = t * topk + min(s0 + j, topk - 1);
                ee[j] = s_ids[p];
                ww[j] = s_rw[p];
#pragma unroll
                for (int cc = 0; cc < kMoeWaves; ++cc)
                    zr[j][cc] = red[((size_t)min(cc, nwc - 1) * 8 + rw) * P + p];
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float z = 0.0f;
#pragma unroll
                for (int cc = 0; cc < kMoeWaves; ++cc) z = cc < nwc ? z + zr[j][cc] : z;
                v = s0 + j < topk && ee[j] >= 0 && ee[j] < E ? fmaf(ww[j], z, v) : v;
            }
        }
        A.y[(int64_t)t * N + n] = v;
    }
}

// Dynamic LDS of moe_down_rows_kernel.
size_t rows_lds_bytes(int P, int E, int nwc, int nw) {
    return align16(sizeof(int) * (((size_t)(P + 3) & ~size_t(3)) + (size_t)E + 2 * (size_t)P)) +
           align16(sizeof(float) * (size_t)nwc * 8 * P) + (size_t)nw * kRowsChunk * kStageBytes;
}

// The tokens' Q8 rows (workgroups 0 .. qgrid-1: q4k_quantize_act's mapping
// and arithmetic, 8 lanes per 32-value block, so the same codes) and, in the
// last workgroup, the call's pair grouping for the gate|up launch: slot a is
// the a-th smallest touched expert (tab_e[a], -1 for the slots past them) and
// its pairs are tab_p[tab_s[a] .. tab_s[a + 1]) -- made once here instead of
// in every workgroup of that launch.  The order of an expert's pairs is free
// (each pair's products are independent of it).
__global__ __launch_bounds__(256) void moe_quantize_group_kernel(
    const float *__restrict__ x, int64_t nblocks, int8_t *__restrict__ codes,
    float *__restrict__ scales, int32_t *__restrict__ sums, const int32_t *__restrict__ ids,
    int P, int E, int slots, int *tab_e, int *tab_s, int *tab_p) {
    extern __shared__ __attribute__((aligned(16))) int lds_g[];
    __shared__ int s_wt[4];
    __shared__ int s_tot[2];
    if ((int)blockIdx.x + 1 < (int)gridDim.x) {
        const int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
        const int sub = threadIdx.x & 7;
        if (blk >= nblocks) return;                // whole 8-lane groups
        const int64_t off = blk * 32 + sub * 4;
        const Q8Lane q = quantize_block8(*reinterpret_cast<const f32x4 *>(x + off));
        *reinterpret_cast<unsigned *>(codes + off) = q.codes;
        if (sub == 0) {
            scales[blk] = q.d;
            sums[blk] = q.sum;
        }
        return;
    }
    const int tid = threadIdx.x, nt = blockDim.x, lane = tid & 63, wave = tid >> 6;
    int *s_ids = lds_g;                            // [P]
    int *cnt = s_ids + P;                          // [E] pairs per expert, then cursor
    for (int p = tid; p < P; p += nt) s_ids[p] = ids[p];
    for (int e = tid; e < E; e += nt) cnt[e] = 0;
    __syncthreads();
    for (int p = tid; p < P; p += nt) {
        const int e = s_ids[p];
        if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    {
        // one scan of (pairs, touched) over expert ranges: each touched expert's
        // slot and first pair
        const int per = (E + nt - 1) / nt;
        const int e0 = min(E, tid * per), e1 = min(E, e0 + per);
        int c = 0, f = 0;
        for (int e = e0; e < e1; ++e) {
            c += cnt[e];
            f += cnt[e] > 0;
        }
        int wtot;
        const int ex = wave_exclusive_scan((c << 16) | f, &wtot);   // c, f <= 4096
        if (lane == 0) s_wt[wave] = wtot;
        __syncthreads();
        int base = ex;
        for (int k = 0; k < wave; ++k) base += s_wt[k];
        int bc = base >> 16, bf = base & 0xFFFF;
        for (int e = e0; e < e1; ++e) {
            const int n = cnt[e];
            if (n > 0) {
                tab_e[bf] = e;
                tab_s[bf] = bc;
                ++bf;
            }
            cnt[e] = bc;
            bc += n;
        }
        if (tid == nt - 1) {
            s_tot[0] = bf;
            s_tot[1] = bc;
        }
    }
    __syncthreads();
    for (int a = s_tot[0] + tid; a < slots; a += nt) tab_e[a] = -1;
    for (int a = s_tot[0] + tid; a <= slots; a += nt) tab_s[a] = s_tot[1];
    for (int p = tid; p < P; p += nt) {
        const int e = s_ids[p];
        if (e >= 0 && e < E) tab_p[atomicAdd(&cnt[e], 1)] = p;
    }
}

// Launch shape for K = 256*nsb: column slots per wave enough that at most
// kMoeWaves waves cover K in one pass (S = kStageSlots at most; wider K takes
// several passes).  The shape depends on K alone -- not on the activation
// form -- so the fused layer and the unfused chain add in the same order.
struct Shape {
    int lg_rg, S, nw, RB;
};
Shape shape(int64_t nsb) {
    Shape s;
    s.lg_rg = 3;
    while ((8 >> s.lg_rg) < kStageSlots &&
           (nsb + (8 >> s.lg_rg) - 1) / (8 >> s.lg_rg) > kMoeWaves)
        --s.lg_rg;
    s.S = 8 >> s.lg_rg;
    s.nw = (int)std::min<int64_t>(kMoeWaves, (nsb + s.S - 1) / s.S);
    s.RB = (1 << s.lg_rg) * kMoeV;
    return s;
}

// Pairs per pass: an expert has at most T pairs when each token lists
// distinct experts, so small T needs no wider pass (more pairs only take more
// passes, the weights then coming from L2).
template <int MODE>
hipError_t launch_kernel(const MoeArgs &A, int64_t T, int nmat, const Shape &sh,
                         hipStream_t stream) {
    dim3 grid((unsigned)((A.N + sh.RB - 1) / sh.RB),
              (unsigned)(nmat * A.slots + A.zero_skipped));
    auto go = [&](auto kern, int MC) {
        hipLaunchKernelGGL(kern, grid, dim3(64 * sh.nw),
                           moe_lds_bytes(A.P, A.E, sh.nw, sh.S, MC), stream, A);
    };
    if constexpr (MODE == ACT_F32_H8) {
        // one token: a workgroup holds RB/2 rows of both projections
        const dim3 g8((unsigned)((A.N + sh.RB / 2 - 1) / (sh.RB / 2)), (unsigned)A.slots);
        hipLaunchKernelGGL((moe_kernel<kMoeV, 1, MODE>), g8, dim3(64 * sh.nw),
                           moe_lds_bytes(A.P, A.E, sh.nw, sh.S, 1), stream, A);
    } else {
        if (T == 1)
            go(moe_kernel<kMoeV, 1, MODE>, 1);
        else if (T <= kMoeMC2MaxT)
            go(moe_kernel<kMoeV, 2, MODE>, 2);
        else
            go(moe_kernel<kMoeV, kMoeMC, MODE>, kMoeMC);
    }
    return hipGetLastError();
}

size_t f32_bytes(int64_t rows, int64_t cols) {
    return (size_t)((4 * rows * cols + 255) & ~int64_t(255));
}

// Routed-sum counters at the front of a workspace: one per row block of an
// N-row launch (row blocks hold at least 16 rows).
size_t counter_bytes(int64_t N) { return f32_bytes(1, (N + 15) / 16); }

}  // namespace

size_t moe_workspace_bytes(int64_t T, int64_t topk, int64_t n_experts, int64_t N) {
    (void)n_experts;
    return counter_bytes(N) + f32_bytes(T * topk, N);   // counters, per-slot products z
}

hipError_t launch_moe_gemv(const uint8_t *w, int64_t n_experts, int64_t stride, int64_t N,
                           int64_t K, const int32_t *ids, const float *route_w, int64_t T,
                           int64_t topk, const int8_t *codes, const float *scales,
                           const int32_t *sums, int act_per_slot, float *y, void *workspace,
                           hipStream_t stream) {
    float *z = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + counter_bytes(N));
    const int P = (int)(T * topk), E = (int)n_experts;
    const Shape sh = shape(K / kQK);
    MoeArgs A = {};
    A.w[0] = A.w[1] = w;
    A.out[0] = A.out[1] = route_w ? z : y;
    A.stride = stride;
    A.N = (int)N;
    A.nsb = (int)(K / kQK);
    A.lg_rg = sh.lg_rg;
    A.topk = (int)topk;
    A.act_per_slot = act_per_slot;
    A.P = P;
    A.E = E;
    A.slots = P < E ? P : E;
    A.zero_skipped = route_w ? 0 : 1;
    A.codes = codes;
    A.scales = scales;
    A.sums = sums;
    A.ids = ids;
    A.direct = T == 1;
    if (route_w) {
        A.route_w = route_w;
        A.y = y;
        A.T = (int)T;
        A.cnt = static_cast<unsigned *>(workspace);
    }
    return launch_kernel<ACT_Q8>(A, T, 1, sh, stream);
}

// Q8 rows: codes, scales, sums (each 256-byte aligned).
size_t q8_rows_bytes(int64_t rows, int64_t K) {
    return f32_bytes(rows, K / 4) + 2 * f32_bytes(rows, K / 32);
}

size_t moe_ffn_workspace_bytes(int64_t T, int64_t topk, int64_t H, int64_t F) {
    const int64_t P = T * topk;
    // counters of the down launch; g, u, z; Q8 of x and of h for the unfused
    // activations of larger T; the pair grouping (3P + 1 ints)
    return counter_bytes(H) + 2 * f32_bytes(P, F) + f32_bytes(P, H) + q8_rows_bytes(T, H) +
           q8_rows_bytes(P, F) + f32_bytes(1, 3 * P + 1);
}

hipError_t launch_moe_ffn(const uint8_t *w_gate, const uint8_t *w_up, const uint8_t *w_down,
                          int64_t n_experts, int64_t stride_gu, int64_t stride_down, int64_t H,
                          int64_t F, const int32_t *ids, const float *route_w, int64_t T,
                          int64_t topk, const float *x, float *y, void *workspace,
                          hipStream_t stream) {
    const int64_t P = T * topk;
    unsigned *cnt = static_cast<unsigned *>(workspace);
    uint8_t *ws = static_cast<uint8_t *>(workspace) + counter_bytes(H);
    float *g = reinterpret_cast<float *>(ws);
    float *u = reinterpret_cast<float *>(ws + f32_bytes(P, F));
    float *z = reinterpret_cast<float *>(ws + 2 * f32_bytes(P, F));
    uint8_t *q8 = ws + 2 * f32_bytes(P, F) + f32_bytes(P, H);
    int8_t *xc = reinterpret_cast<int8_t *>(q8);
    float *xs = reinterpret_cast<float *>(q8 + f32_bytes(T, H / 4));
    int32_t *xsu = reinterpret_cast<int32_t *>(q8 + f32_bytes(T, H / 4) + f32_bytes(T, H / 32));
    uint8_t *hq = q8 + q8_rows_bytes(T, H);
    int8_t *hc = reinterpret_cast<int8_t *>(hq);
    float *hs = reinterpret_cast<float *>(hq + f32_bytes(P, F / 4));
    int32_t *hsu = reinterpret_cast<int32_t *>(hq + f32_bytes(P, F / 4) + f32_bytes(P, F / 32));
    int *tab = reinterpret_cast<int *>(hq + q8_rows_bytes(P, F));   // [P] e, [P + 1] s, [P] p
    const int E = (int)n_experts;
    const Shape sh1 = shape(H / kQK), sh2 = shape(F / kQK);
    // gate|up forming Q8(h) itself: each workgroup holds the same rows of both
    // projections for one pair (slot a = pair a, a token's repeated expert
    // computed twice with the same bits); RG = 8 rows per lane group and one
    // column per wave, as many waves as sh1 covers columns per pass, so a lane
    // adds the same columns in the same order as under sh1 and g, u keep the
    // gate|up launch's own bits
    auto gate_up_h8 = [&]() {
        MoeArgs A = {};
        A.w[0] = w_gate;
        A.w[1] = w_up;
        A.out[0] = g;
        A.out[1] = u;
        A.stride = stride_gu;
        A.N = (int)F;
        A.nsb = (int)(H / kQK);
        A.topk = (int)topk;
        A.P = (int)P;
        A.E = E;
        A.slots = (int)P;
        A.ids = ids;
        A.direct = 1;
        A.xa = x;
        A.hc = hc;
        A.hs = hs;
        A.hsu = hsu;
        Shape sh8;
        sh8.lg_rg = 3;
        sh8.S = 1;
        sh8.nw = sh1.nw * sh1.S;
        sh8.RB = 8 * kMoeV;
        A.lg_rg = sh8.lg_rg;
        return launch_kernel<ACT_F32_H8>(A, T, 1, sh8, stream);
    };
    // down on the prepared Q8(h) with the routed sum inside each workgroup
    MoeArgs B = {};
    B.w[0] = w_down;
    B.stride = stride_down;
    B.N = (int)H;
    B.nsb = (int)(F / kQK);
    B.topk = (int)topk;
    B.P = (int)P;
    B.E = E;
    B.ids = ids;
    B.codes = hc;
    B.scales = hs;
    B.sums = hsu;
    B.act_per_slot = 1;
    B.route_w = route_w;
    B.y = y;
    B.T = (int)T;
    const dim3 down_grid((unsigned)((H + 7) / 8));
    if (T == 1 && topk <= kDownSumSlots && sh2.lg_rg == 3) {
        // One token: no grouping at all; the down workgroups hold every slot's
        // weights at once.  Same bits as the launches below.
        hipError_t err = gate_up_h8();
        if (err != hipSuccess) return err;
        // up to 4 slots: one set of waves; up to 8: two sets of 4 slots
        if (topk <= 4)
            hipLaunchKernelGGL((moe_down_sum_kernel<4, 4>), down_grid, dim3(64 * sh2.nw), 0, stream, B);
        else
            hipLaunchKernelGGL((moe_down_sum_kernel<kDownSumSlots, 4>), down_grid,
                               dim3(2 * 64 * sh2.nw), 0, stream, B);
        return hipGetLastError();
    }
    if (T > 1 && P <= kRowsMaxPairs && sh2.lg_rg == 3) {
        // A few tokens: Q8(h) from the gate|up launch (two tokens) or the
        // quantizer (more), then one down launch over every pair per row
        // block that sums the slots in the workgroup.  Same bits.
        hipError_t err;
        if (T <= kFuseMaxT) {
            err = gate_up_h8();
        } else {
            // x's Q8 rows and the pair grouping in one launch
            const int slots = (int)(P < E ? P : E);
            const int64_t nblocks = T * (H / kQB);
            const int qgrid = (int)((nblocks + 31) / 32);
            hipLaunchKernelGGL(moe_quantize_group_kernel, dim3(qgrid + 1), dim3(256),
                               sizeof(int) * (size_t)(P + E), stream, x, nblocks, xc, xs, xsu,
                               ids, (int)P, E, slots, tab, tab + P, tab + 2 * P + 1);
            err = hipGetLastError();
            if (err != hipSuccess) return err;
            MoeArgs A = {};
            A.tab_e = tab;
            A.tab_s = tab + P;
            A.tab_p = tab + 2 * P + 1;
            A.w[0] = w_gate;
            A.w[1] = w_up;
            A.out[0] = g;
            A.out[1] = u;
            A.stride = stride_gu;
            A.N = (int)F;
            A.nsb = (int)(H / kQK);
            A.lg_rg = sh1.lg_rg;
            A.topk = (int)topk;
            A.P = (int)P;
            A.E = E;
            A.slots = (int)(P < E ? P : E);
            A.ids = ids;
            A.codes = xc;
            A.scales = xs;
            A.sums = xsu;
            err = launch_kernel<ACT_Q8>(A, T, 2, sh1, stream);
            if (err != hipSuccess) return err;
            err = launch_quantize(u, P, F, g, hc, hs, hsu, stream);
        }
        if (err != hipSuccess) return err;
        const int nwc = sh2.nw, nw = nwc * (16 / nwc);
        hipLaunchKernelGGL((moe_down_rows_kernel<kRowsChunk>), down_grid, dim3(64 * nw),
                           rows_lds_bytes((int)P, E, nwc, nw), stream, B);
        return hipGetLastError();
    }
    // In-kernel activations quantize a token's row once per workgroup that
    // reads it (row blocks x experts); past a few tokens that repetition costs
    // more than the launches a separate quantizer needs.  Same codes either way.
    const bool fuse = T <= kFuseMaxT;
    // gate and up in one launch
    MoeArgs A = {};
    A.w[0] = w_gate;
    A.w[1] = w_up;
    A.out[0] = g;
    A.out[1] = u;
    A.stride = stride_gu;
    A.N = (int)F;
    A.nsb = (int)(H / kQK);
    A.lg_rg = sh1.lg_rg;
    A.topk = (int)topk;
    A.act_per_slot = 0;
    A.P = (int)P;
    A.E = E;
    A.slots = (int)(P < E ? P : E);
    A.zero_skipped = 0;
    A.ids = ids;
    A.direct = T == 1;
    hipError_t err;
    if (fuse) {
        A.xa = x;
        err = launch_kernel<ACT_F32>(A, T, 2, sh1, stream);
    } else {
        err = launch_quantize(x, T, H, nullptr, xc, xs, xsu, stream);
        if (err != hipSuccess) return err;
        A.codes = xc;
        A.scales = xs;
        A.sums = xsu;
        err = launch_kernel<ACT_Q8>(A, T, 2, sh1, stream);
    }
    if (err != hipSuccess) return err;
    // down: SwiGLU(g, u) quantized in the kernel, per-slot products z, and the
    // routed sum by the last workgroup of each row block
    B = A;
    B.route_w = route_w;
    B.y = y;
    B.T = (int)T;
    B.cnt = cnt;
    B.w[0] = B.w[1] = w_down;
    B.out[0] = B.out[1] = z;
    B.stride = stride_down;
    B.N = (int)H;
    B.nsb = (int)(F / kQK);
    B.lg_rg = sh2.lg_rg;
    B.act_per_slot = 1;
    if (fuse) {
        B.xa = g;
        B.xb = u;
        err = launch_kernel<ACT_SWIGLU>(B, T, 1, sh2, stream);
    } else {
        err = launch_quantize(u, P, F, g, hc, hs, hsu, stream);
        if (err != hipSuccess) return err;
        B.codes = hc;
        B.scales = hs;
        B.sums = hsu;
        err = launch_kernel<ACT_Q8>(B, T, 1, sh2, stream);
    }
    return err;
}

}  // namespace q4k
