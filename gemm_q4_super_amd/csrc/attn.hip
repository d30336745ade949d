// INT8 KV cache and decode attention over it.
//
// Cache format (genie-ai-runtime's Path I, section 4 "Memory-first: making
// every byte count"): every (layer, position, kv-head) vector of 128 values is
// stored as int8 codes with one fp32 absmax scale, scale = fl32(amax / 127),
// code = rne(fl32(x / scale)).  One layer's cache is head-major,
//   codes int8 [n_kv][cap][128], scales fp32 [n_kv][cap]  (K and V alike),
// so the positions of one kv head are a contiguous stream.
//
// kv_store_kernel: one wave per new vector, lane l holding values 2l, 2l+1;
// the scale and the quotients are the correctly rounded ones of the Q8
// activation quantizer (same helpers), so codes match IEEE division bit for bit.
//
// attn_kernel: decode attention of M query tokens with grouped kv heads
// (query head h reads kv head h / G).  The problem is a stream of
// n_kv * n_ctx * 256 bytes of codes plus 8 bytes of scales per position and
// head, against 4 multiply-adds per byte per query vector: HBM-bound at one
// token, so the design is about keeping enough loads in flight, not about the
// matrix cores.
//  * Work unit: (kv head, block of 4 query vectors, chunk of positions).  A
//    query vector is (token m, head g of the group), index v = m*G + g.  The
//    K and V bytes of a chunk are read once for the 4 vectors.
//  * Lanes: lane = 8*j + s reads the 16 bytes s of position 8*pass + j, so a
//    wave load covers 8 whole positions (1 KB contiguous).  Positions come in
//    rounds of 4 passes (32 positions per wave); two waves per SIMD overlap
//    one's loads with the other's arithmetic.
//  * Scores in base 2: s = (sum_i q_i * k_i) * (kscale * scale * log2 e); the
//    int8 code k is read as the unsigned byte u = k + 128 (one conversion per
//    byte), and the bias is taken out once per lane: sum q_i u_i - 128 sum q_i.
//    The 8 lanes of a position add their partial dots (DPP).
//  * Softmax: each lane keeps a running max, the running sums of p and of
//    p * vscale, and its 16 output dims of sum p * vscale * u (online
//    rescaling when the max grows).  At the end lanes j and j^1 merge (DPP),
//    and the 4 partials per wave of the workgroup merge through LDS, giving one
//    partial (o[128], max, sum) per query vector and chunk.  No reduction
//    goes through cross-lane permutes, whose latency would chain.
//  * Chunks are merged in chunk order by the last workgroup of the unit to
//    finish (a per-unit counter in the workspace, returned to zero), so the
//    result does not depend on the order the workgroups ran in.  With one
//    chunk the workgroup writes the output directly.
#include <math.h>

#include <type_traits>

#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kHD = 128;         // head dimension
constexpr int kQV = 4;           // query vectors per workgroup
constexpr int kWaves = 8;        // waves per workgroup
constexpr int kRound = 32;       // positions per wave round (4 passes of 8)
constexpr int kPartStride = 132; // floats per (chunk, query vector) partial: o[128], max, sum
constexpr int kRowRotate8 = 0x128;   // DPP row_ror:8: lane i <-> i^8 within 16 lanes

// ------------------------------------------------------------- cache store --

__global__ __launch_bounds__(256) void kv_store_kernel(const float *__restrict__ k,
                                                      const float *__restrict__ v, int M, int n_kv,
                                                      int64_t pos0, int64_t cap,
                                                      int8_t *__restrict__ kc,
                                                      float *__restrict__ ks,
                                                      int8_t *__restrict__ vc,
                                                      float *__restrict__ vs) {
    const int lane = threadIdx.x & 63;
    const int vec = blockIdx.x * 4 + (threadIdx.x >> 6);   // ((m * n_kv + h) * 2 + which)
    if (vec >= M * n_kv * 2) return;
    const int which = vec & 1, mh = vec >> 1;
    const int m = mh / n_kv, h = mh % n_kv;
    const float *src = (which ? v : k) + (int64_t)mh * kHD;
    const float2 x = reinterpret_cast<const float2 *>(src)[lane];
    unsigned a = max(__float_as_uint(x.x) & 0x7FFFFFFFu, __float_as_uint(x.y) & 0x7FFFFFFFu);
    a = max(a, (unsigned)dpp_i<kQuadSwap1>((int)a));
    a = max(a, (unsigned)dpp_i<kQuadSwap2>((int)a));
    a = max(a, (unsigned)dpp_i<kRowHalfMirror>((int)a));
    a = max(a, (unsigned)__shfl_xor((int)a, 8));
    a = max(a, (unsigned)__shfl_xor((int)a, 16));
    a = max(a, (unsigned)__shfl_xor((int)a, 32));
    const float d = q8_scale(__uint_as_float(a));
    const float dd = d == 0.0f ? 1.0f : d;   // all-zero vector: codes 0
    float q0, q1;
    if (__builtin_amdgcn_ballot_w64(dd < 0x1p-100f) != 0) {
        q0 = __builtin_amdgcn_fmed3f(x.x / dd, -127.0f, 127.0f);
        q1 = __builtin_amdgcn_fmed3f(x.y / dd, -127.0f, 127.0f);
    } else {
        const float r1 = q8_recip(dd);
        q0 = q8_quotient(x.x, dd, r1);
        q1 = q8_quotient(x.y, dd, r1);
    }
    // rne by the 1.5 * 2^23 shift: the code sits in the low mantissa bits
    const unsigned b0 = __float_as_uint(q0 + 0x1.8p23f) & 0xFFu;
    const unsigned b1 = __float_as_uint(q1 + 0x1.8p23f) & 0xFFu;
    const int64_t row = (int64_t)h * cap + pos0 + m;
    int8_t *dst = (which ? vc : kc) + row * kHD;
    reinterpret_cast<unsigned short *>(dst)[lane] = (unsigned short)(b0 | (b1 << 8));
    if (lane == 0) (which ? vs : ks)[row] = d;
}

// --------------------------------------------------------------- attention --

struct AttnArgs {
    const float *q;      // [M][n_head][128]
    const int8_t *kc;    // [n_kv][cap][128]
    const float *ks;     // [n_kv][cap]
    const int8_t *vc;
    const float *vs;
    float *out;          // [M][n_head][128]
    unsigned *cnt;       // [units], zero between calls
    float *part;         // [units][n_chunks][4][kPartStride]
    int64_t cap;
    int n_ctx, M, G, n_kv, nqb, chunk, n_chunks;
    float scale_log2;    // softmax scale times log2(e)
};

__device__ __forceinline__ void bytes_to_float(const u32x4 raw, float u[16]) {
    // code + 128 as an unsigned byte, converted exactly
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const unsigned b = raw[w] ^ 0x80808080u;
        u[4 * w + 0] = (float)(b & 0xFFu);          // v_cvt_f32_ubyte0..3
        u[4 * w + 1] = (float)((b >> 8) & 0xFFu);
        u[4 * w + 2] = (float)((b >> 16) & 0xFFu);
        u[4 * w + 3] = (float)(b >> 24);
    }
}

__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }

// exp2(m_old - m_new) for m_new >= m_old, 1 when both are -inf (nothing seen).
__device__ __forceinline__ float rescale(float m_old, float m_new) {
    return m_old == m_new ? 1.0f : exp2_f(m_old - m_new);
}

struct Round {
    u32x4 k[4], v[4];
    float ks[4], vs[4];
};

__global__ __launch_bounds__(64 * kWaves) void attn_kernel(const AttnArgs a) {
    __shared__ float red[kWaves][4][kQV][kPartStride];   // [wave][lane row][r][...]
    __shared__ float fac[kQV][kWaves * 4], fac_max[kQV];
    __shared__ unsigned last_flag;
    const int units = a.n_kv * a.nqb;
    const int unit = blockIdx.x % units;      // neighbouring workgroups: different units
    const int chunk = blockIdx.x / units;
    const int kvh = unit / a.nqb, qb = unit % a.nqb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int j = lane >> 3, sg = lane & 7;
    const int GM = a.G * a.M;
    const int n_head = a.G * a.n_kv;

    const int per_wave = a.chunk / kWaves;
    const int t_begin = chunk * a.chunk + wave * per_wave;
    const int t_end = min(t_begin + per_wave, a.n_ctx);
    const int8_t *kb = a.kc + (int64_t)kvh * a.cap * kHD + sg * 16;
    const int8_t *vb = a.vc + (int64_t)kvh * a.cap * kHD + sg * 16;
    const float *ksb = a.ks + (int64_t)kvh * a.cap;
    const float *vsb = a.vs + (int64_t)kvh * a.cap;

    auto load_round = [&](int tb, Round &R) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int t = tb + 8 * p + j;
            if (t < t_end) {
                R.k[p] = *reinterpret_cast<const u32x4 *>(kb + (int64_t)t * kHD);
                R.v[p] = *reinterpret_cast<const u32x4 *>(vb + (int64_t)t * kHD);
                R.ks[p] = ksb[t];
                R.vs[p] = vsb[t];
            } else {
                R.k[p] = u32x4{0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
                R.v[p] = R.k[p];
                R.ks[p] = 0.0f;
                R.vs[p] = 0.0f;
            }
        }
    };

    // The first round's loads go out before the query vectors are read, so
    // the two latencies overlap.
    Round first;
    if (t_begin < t_end) load_round(t_begin, first);

    // The 16 dims sg*16.. of the block's query vectors, and their sums.
    float qr[kQV][16], qsum[kQV];
    int vis[kQV];
#pragma unroll
    for (int r = 0; r < kQV; ++r) {
        const int v = qb * kQV + r;
        if (v < GM) {
            const int m = v / a.G, g = v % a.G;
            const float4 *src = reinterpret_cast<const float4 *>(
                a.q + ((int64_t)m * n_head + kvh * a.G + g) * kHD + sg * 16);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float4 t = src[w];
                qr[r][4 * w] = t.x;
                qr[r][4 * w + 1] = t.y;
                qr[r][4 * w + 2] = t.z;
                qr[r][4 * w + 3] = t.w;
            }
            vis[r] = a.n_ctx - (a.M - 1 - m);
        } else {
#pragma unroll
            for (int i = 0; i < 16; ++i) qr[r][i] = 0.0f;
            vis[r] = 0;
        }
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += qr[r][i];
        qsum[r] = sum;
    }

    float m_run[kQV], l_run[kQV], w_run[kQV], acc[kQV][16];
#pragma unroll
    for (int r = 0; r < kQV; ++r) {
        m_run[r] = -INFINITY;
        l_run[r] = 0.0f;
        w_run[r] = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[r][i] = 0.0f;
    }

    // One round: scores of up to 4 passes, the online-softmax update, and the
    // values.  FULL: all 4 passes hold positions of the range (no pass test,
    // so the 4 passes schedule as one block).
    auto round_step = [&](const Round &cur, int tb, auto full) {
        constexpr bool FULL = decltype(full)::value;
        const int npass = FULL ? 4 : min(4, (t_end - tb + 7) >> 3);
        float s[kQV][4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (!FULL && p >= npass) {
#pragma unroll
                for (int r = 0; r < kQV; ++r) s[r][p] = -INFINITY;
                continue;
            }
            float u[16];
            bytes_to_float(cur.k[p], u);
            const int t = tb + 8 * p + j;
            const float f = cur.ks[p] * a.scale_log2;
#pragma unroll
            for (int r = 0; r < kQV; ++r) {
                float d = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) d = fmaf(qr[r][i], u[i], d);
                d = group8_sum(fmaf(-128.0f, qsum[r], d));
                s[r][p] = (t < t_end && t < vis[r]) ? d * f : -INFINITY;
            }
        }
#pragma unroll
        for (int r = 0; r < kQV; ++r) {
            const float mx = fmaxf(fmaxf(s[r][0], s[r][1]), fmaxf(s[r][2], s[r][3]));
            const float mn = fmaxf(m_run[r], mx);
            const float al = rescale(m_run[r], mn);
            m_run[r] = mn;
            l_run[r] *= al;
            w_run[r] *= al;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[r][i] *= al;
        }
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            if (!FULL && p >= npass) break;
            float u[16];
            bytes_to_float(cur.v[p], u);
#pragma unroll
            for (int r = 0; r < kQV; ++r) {
                const float pr = s[r][p] == -INFINITY ? 0.0f : exp2_f(s[r][p] - m_run[r]);
                l_run[r] += pr;
                const float w = pr * cur.vs[p];
                w_run[r] += w;
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[r][i] = fmaf(w, u[i], acc[r][i]);
            }
        }
    };

    // The other wave of the SIMD hides a round's load latency (prefetching
    // the next round into registers measured no faster).
    auto do_round = [&](const Round &cur, int tb) {
        if (tb + kRound <= t_end)
            round_step(cur, tb, std::true_type());
        else
            round_step(cur, tb, std::false_type());
    };
    if (t_begin < t_end) {
        do_round(first, t_begin);
        for (int tb = t_begin + kRound; tb < t_end; tb += kRound) {
            Round cur;
            load_round(tb, cur);
            do_round(cur, tb);
        }
    }

    // Take the +128 bias out and merge position lanes j and j^1 (DPP within a
    // 16-lane row); the even j then hold 4 partials per wave.
#pragma unroll
    for (int r = 0; r < kQV; ++r) {
        const float mo = dpp_f<kRowRotate8>(m_run[r]);
        const float mw = fmaxf(m_run[r], mo);
        const float f = rescale(m_run[r], mw), fo = rescale(mo, mw);
        l_run[r] = l_run[r] * f + dpp_f<kRowRotate8>(l_run[r]) * fo;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float x = fmaf(-128.0f, w_run[r], acc[r][i]);
            acc[r][i] = x * f + dpp_f<kRowRotate8>(x) * fo;
        }
        m_run[r] = mw;
    }
    if ((j & 1) == 0) {
        const int row = j >> 1;
#pragma unroll
        for (int r = 0; r < kQV; ++r) {
            float4 *d4 = reinterpret_cast<float4 *>(&red[wave][row][r][sg * 16]);
#pragma unroll
            for (int w = 0; w < 4; ++w)
                d4[w] = make_float4(acc[r][4 * w], acc[r][4 * w + 1], acc[r][4 * w + 2], acc[r][4 * w + 3]);
            if (sg == 0) {
                red[wave][row][r][kHD] = m_run[r];
                red[wave][row][r][kHD + 1] = l_run[r];
            }
        }
    }
    __syncthreads();

    // Merge the workgroup's partials (4 per wave).  The rescale factors
    // 2^(m_e - max) are formed once per (query vector, partial) into LDS; then
    // thread (r, dims c0..c0+kDims-1) sums its outputs.
    constexpr int kE = kWaves * 4;
    constexpr int kDims = kQV * kHD / (64 * kWaves);   // consecutive dims per thread
    static_assert(kDims == 1 || kDims == 2, "threads per query block");
    if (threadIdx.x < kQV * kE) {
        const int fr = threadIdx.x / kE, fe = threadIdx.x % kE;
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < kE; ++e) mx = fmaxf(mx, red[e >> 2][e & 3][fr][kHD]);
        fac[fr][fe] = rescale(red[fe >> 2][fe & 3][fr][kHD], mx);
        if (fe == 0) fac_max[fr] = mx;
    }
    __syncthreads();
    const int r = threadIdx.x / (kHD / kDims), c0 = (threadIdx.x % (kHD / kDims)) * kDims;
    const float mc = fac_max[r];
    float o[kDims], lc = 0.0f;
#pragma unroll
    for (int d = 0; d < kDims; ++d) o[d] = 0.0f;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const float *pe = red[e >> 2][e & 3][r];
        const float f = fac[r][e];
#pragma unroll
        for (int d = 0; d < kDims; ++d) o[d] = fmaf(f, pe[c0 + d], o[d]);
        lc = fmaf(f, pe[kHD + 1], lc);
    }
    const int v = qb * kQV + r;
    const bool valid = v < GM;
    float *dst = valid ? a.out + ((int64_t)(v / a.G) * n_head + kvh * a.G + v % a.G) * kHD + c0
                       : nullptr;
    if (a.n_chunks == 1) {
        if (valid)
#pragma unroll
            for (int d = 0; d < kDims; ++d) dst[d] = o[d] / lc;
        return;
    }

    // Partial of this chunk, through agent-coherent stores; the counter is
    // bumped once every store of the workgroup has completed.
    float *pp = a.part + (((int64_t)unit * a.n_chunks + chunk) * kQV + r) * kPartStride;
#pragma unroll
    for (int d = 0; d < kDims; ++d)
        __hip_atomic_store(pp + c0 + d, o[d], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (c0 == 0)
        __hip_atomic_store(reinterpret_cast<unsigned long long *>(pp + kHD),
                           (unsigned long long)__float_as_uint(mc) |
                               ((unsigned long long)__float_as_uint(lc) << 32),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0)
        last_flag = __hip_atomic_fetch_add(a.cnt + unit, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(a.n_chunks - 1);
    __syncthreads();
    if (!last_flag) return;

    // The last workgroup of the unit merges the chunks in chunk order; every
    // thread loads every chunk's (max, sum) and its dims before using any.
    const float *pu = a.part + (int64_t)unit * a.n_chunks * kQV * kPartStride + r * kPartStride;
    unsigned long long ml[kMaxAttnChunks];
    float od[kMaxAttnChunks][kDims];
#pragma unroll
    for (int k = 0; k < kMaxAttnChunks; ++k)
        if (k < a.n_chunks) {
            const float *pc = pu + (int64_t)k * kQV * kPartStride;
            ml[k] = __hip_atomic_load(reinterpret_cast<const unsigned long long *>(pc + kHD),
                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
            for (int d = 0; d < kDims; ++d)
                od[k][d] = __hip_atomic_load(pc + c0 + d, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    float mall = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMaxAttnChunks; ++k)
        if (k < a.n_chunks) mall = fmaxf(mall, __uint_as_float((unsigned)ml[k]));
    float lsum = 0.0f;
#pragma unroll
    for (int d = 0; d < kDims; ++d) o[d] = 0.0f;
#pragma unroll
    for (int k = 0; k < kMaxAttnChunks; ++k)
        if (k < a.n_chunks) {
            const float f = rescale(__uint_as_float((unsigned)ml[k]), mall);
            lsum = fmaf(f, __uint_as_float((unsigned)(ml[k] >> 32)), lsum);
#pragma unroll
            for (int d = 0; d < kDims; ++d) o[d] = fmaf(f, od[k][d], o[d]);
        }
    if (valid)
#pragma unroll
        for (int d = 0; d < kDims; ++d) dst[d] = o[d] / lsum;
    if (threadIdx.x == 0) __hip_atomic_store(a.cnt + unit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Chunking: about kAttnTargetGroups workgroups in all, chunks a multiple of
// one wave round per wave, at most kMaxAttnChunks per unit, and at least
// n_ctx/8 positions up to 256: the last workgroup's chunk-ordered merge grows
// with the chunk count, so a short context is better cut into fewer, longer
// chunks (Qwen3-4B heads, one token: 2048 positions 14.9 -> 12.7 us, 4096
// 16.3 -> 14.3 us, 1024 11.8 -> 11.4 us; unchanged from 8192 on).
struct AttnPlan {
    int nqb, units, chunk, n_chunks;
};

AttnPlan plan_attn(int64_t M, int64_t n_head, int64_t n_kv, int64_t n_ctx) {
    AttnPlan p;
    const int64_t GM = (n_head / n_kv) * M;
    p.nqb = (int)((GM + kQV - 1) / kQV);
    p.units = (int)(n_kv * p.nqb);
    const int64_t step = (int64_t)kWaves * 8;   // a chunk gives every wave whole passes
    int64_t want = std::max<int64_t>(1, std::min<int64_t>(kMaxAttnChunks, kAttnTargetGroups / p.units));
    int64_t chunk = (n_ctx + want - 1) / want;
    const int64_t lo = std::min<int64_t>(256, (n_ctx / 8 + step - 1) / step * step);
    chunk = std::max<int64_t>(std::max<int64_t>(step, lo), (chunk + step - 1) / step * step);
    p.chunk = (int)chunk;
    p.n_chunks = (int)((n_ctx + chunk - 1) / chunk);
    return p;
}

}  // namespace

size_t attn_workspace_bytes(int64_t M, int64_t n_head, int64_t n_kv) {
    const int64_t GM = (n_head / n_kv) * M;
    const int64_t units = n_kv * ((GM + kQV - 1) / kQV);
    return kAttnCounterBytes + (size_t)units * kMaxAttnChunks * kQV * kPartStride * sizeof(float);
}

hipError_t launch_kv_store(const float *k, const float *v, int64_t M, int64_t n_kv, int64_t pos0,
                           int64_t cap, int8_t *kc, float *ks, int8_t *vc, float *vs,
                           hipStream_t stream) {
    const int64_t vecs = M * n_kv * 2;
    hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)((vecs + 3) / 4)), dim3(256), 0, stream, k,
                       v, (int)M, (int)n_kv, pos0, cap, kc, ks, vc, vs);
    return hipGetLastError();
}

hipError_t launch_attn(const float *q, int64_t M, int64_t n_head, int64_t n_kv, const int8_t *kc,
                       const float *ks, const int8_t *vc, const float *vs, int64_t cap,
                       int64_t n_ctx, float scale, float *out, void *workspace,
                       hipStream_t stream) {
    const AttnPlan p = plan_attn(M, n_head, n_kv, n_ctx);
    AttnArgs a;
    a.q = q;
    a.kc = kc;
    a.ks = ks;
    a.vc = vc;
    a.vs = vs;
    a.out = out;
    a.cnt = static_cast<unsigned *>(workspace);
    a.part = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + kAttnCounterBytes);
    a.cap = cap;
    a.n_ctx = (int)n_ctx;
    a.M = (int)M;
    a.G = (int)(n_head / n_kv);
    a.n_kv = (int)n_kv;
    a.nqb = p.nqb;
    a.chunk = p.chunk;
    a.n_chunks = p.n_chunks;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634);
    hipLaunchKernelGGL(attn_kernel, dim3((unsigned)(p.units * p.n_chunks)), dim3(64 * kWaves), 0,
                       stream, a);
    return hipGetLastError();
}

}  // namespace q4k
