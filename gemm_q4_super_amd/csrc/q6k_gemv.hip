// Q6_K decode / small-batch GEMV: y[M][N] = Q8(x)[M][K] * W^T with W in Q6_K,
// M = 1..8 (the staged Q8 rows within one workgroup's LDS, e.g. M = 8 at
// K = 9728 in the 160 KB of a gfx950 workgroup), on prepared Q8 rows (q6k_gemv) or on fp32 rows that
// each workgroup quantizes with q4k_quantize_act's arithmetic
// (q6k_quantize_gemv: same codes, so the two give the same bits).
//
// Q6_K (public GGUF layout; real Q4_K_M files keep some tensors in it, and the
// decode kernels of genie's "Path G" -- "genie-ai-runtime ...", section 6,
// "The negatives I kept" -- are Q6_K ones): 256 weights of one row in 210 bytes, ql[128] (low 4 bits of
// the 6-bit quants), qh[64] (high 2 bits), int8 sc[16] (one per 16 weights),
// fp16 d; w = d*sc[e/16]*(q[e] - 32).  Element e = 128h + 32t + l keeps its low
// bits in ql[64h + 32(t%2) + l] (low nibble for t < 2, high for t >= 2) and its
// high bits in bits 2t..2t+1 of qh[32h + l].
//
// Bandwidth-bound like the Q4_K decode GEMV; what differs:
//  * Alignment.  210 = 2 (mod 4), so a super-block starts at an even byte.
//    Every load here is 4-byte aligned and stays inside its super-block: an
//    8-byte field at S + o (o = 0 mod 8) is read as the 12 bytes from
//    S + o - (S & 2) and shifted into place (v_alignbyte); the scales take 8
//    bytes from S + 192 + 8h - (S & 2) plus a 2-byte load, d a 2-byte load.
//  * Lane layout.  8 lanes per super-block, lane 4h + u owning elements
//    128h + 32t + 8u + i (t < 4, i < 8): 8 bytes of each of ql[64h + 8u],
//    ql[64h + 32 + 8u], qh[32h + 8u].  Its partial dot for Q8 block j = 4h + t
//    is P = sum_i (q - 32) c over 8 elements (two sdot4 on q in 0..63, plus
//    -32 * sum c, precomputed per activation row when the Q8 rows are staged);
//    the lane adds a_j * (d * sc) * P to its accumulator, sc = sc[8h + 2t + u/2]
//    (the 16-weight sub-block of its 8 elements).
//  * A workgroup: 8 V rows (lane group g of every wave: rows 8v + g), W waves
//    splitting the K/256 columns (CPW per wave); each wave stages the Q8 rows of
//    its own columns in LDS in the lanes' order, issues every weight load of
//    its units before any arithmetic, and the per-lane sums reduce over the 8
//    lanes (DPP) and the waves (LDS, fixed order).
#include <algorithm>

#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kQ6Bytes = 210;
constexpr int kQ6Waves = 16;
// LDS of one staged (column, activation row): 256 codes in lane order, 8 block
// scales, 32 offset terms (-32 * sum of a lane's 8 codes of a block).
constexpr int kQ6Stage = 256 + 32 + 128;

__device__ __forceinline__ u32x4 load12(const uint8_t *p) {   // 4-byte aligned
    const unsigned *q = reinterpret_cast<const unsigned *>(p);
    u32x4 r;
    r.x = q[0];
    r.y = q[1];
    r.z = q[2];
    r.w = 0;
    return r;
}

// One workgroup: rows row_base .. row_base + 8V - 1 of one product.
template <int M, int CPW, int V, bool FUSED>
__device__ __forceinline__ void q6k_rows(
    const uint8_t *__restrict__ w, float *__restrict__ y, const int8_t *__restrict__ codes,
    const float *__restrict__ scales, const float *__restrict__ x, const int N, const int nsb,
    const int row_base) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ float red[kQ6Waves][8 * V][M];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int nw = blockDim.x >> 6;
    const int g = lane >> 3;              // row of the 8-row set
    const int h = (lane >> 2) & 1, u = lane & 3;
    const int K = nsb * 256, nblk = nsb * 8;
    const int wcol0 = wave * CPW;
    const int ncols = min(CPW, nsb - wcol0);   // >= 1 (the host sizes the workgroup)

    // ---- stage this wave's columns: lane-order codes, scales, offset terms.
    // Prepared rows: piece p < 32 of a (column, row) is block j = p/4, quarter
    // u = p%4 (8 codes).  fp32 rows: lane L holds values 4(L%8).. of block L/8
    // (the quantizer's layout).
    const int sp = lane & 31, sj = sp >> 2, su = sp & 3;
    const int sdst = (((sj >> 2) * 4 + su) * 4 + (sj & 3));   // slot of the piece
    constexpr int PC = FUSED ? 1 : (M + 1) / 2;
    constexpr int PX = FUSED ? M : 1;
    uint2 cv[CPW][PC];
    float av[CPW];
    f32x4 xv[CPW][PX];
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int b = min(wcol0 + c, nsb - 1);
        if constexpr (FUSED) {
#pragma unroll
            for (int m = 0; m < M; ++m)
                xv[c][m] = *reinterpret_cast<const f32x4 *>(x + (int64_t)m * K + 256 * b + 4 * lane);
        } else {
#pragma unroll
            for (int k = 0; k < PC; ++k) {
                const int m = min(2 * k + (lane >> 5), M - 1);
                cv[c][k] =
                    *reinterpret_cast<const uint2 *>(codes + (int64_t)m * K + 256 * b + 8 * sp);
            }
            av[c] = scales[(int64_t)min(lane >> 3, M - 1) * nblk + 8 * b + (lane & 7)];
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- weight loads (branch-free: rows past N read row N-1 and are never
    // written; columns past nsb are never added)
    // Addresses: a 4-byte-aligned scalar base at or below the workgroup's first
    // row (w is 16-byte aligned) plus 32-bit offsets, so a super-block's
    // offset and its start address agree mod 4.
    const int64_t row_bytes = (int64_t)nsb * kQ6Bytes;
    const int64_t first = (int64_t)row_base * row_bytes;
    const uint8_t *__restrict__ wb = w + (first & ~int64_t(3));
    const unsigned rem = (unsigned)(first & 3);
    u32x4 qa[V][CPW], qb[V][CPW], qh[V][CPW];
    uint2 qs[V][CPW];
    unsigned qt[V][CPW], qd[V][CPW], qo[V][CPW];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const unsigned rr = (unsigned)(min(row_base + 8 * v + g, N - 1) - row_base);
            const unsigned b = (unsigned)min(wcol0 + c, nsb - 1);
            const unsigned off = rem + rr * (unsigned)row_bytes + b * (unsigned)kQ6Bytes;
            const unsigned odd = off & 2u;   // super-block start = 2 (mod 4)
            const unsigned base = off - odd; // >= 0: off >= rem >= odd for the first one
            qo[v][c] = odd;
            qa[v][c] = load12(wb + (base + 64u * h + 8u * u));
            qb[v][c] = load12(wb + (base + 64u * h + 32u + 8u * u));
            qh[v][c] = load12(wb + (base + 128u + 32u * h + 8u * u));
            qs[v][c] = *reinterpret_cast<const uint2 *>(wb + (base + 192u + 8u * h));
            qt[v][c] = *reinterpret_cast<const unsigned short *>(wb + (off + 198u + 8u * h));
            qd[v][c] = *reinterpret_cast<const unsigned short *>(wb + (off + 208u));
        }
    __builtin_amdgcn_sched_barrier(0);

    // ---- LDS stores of the staged columns ([column][row] stages)
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        if (c >= ncols) continue;   // wave-uniform
        const int b = wcol0 + c;
        if constexpr (FUSED) {
            // quantize: lane L -> block j = L/8, values 4i..4i+3 (i = L%8), i.e.
            // quarter u = i/2, half i%2 of its 8-code piece
            const int j = lane >> 3, i = lane & 7;
            const int slot = ((j >> 2) * 4 + (i >> 1)) * 4 + (j & 3);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const Q8Lane q8 = quantize_block8(xv[c][m]);
                uint8_t *st = lds + ((size_t)b * M + m) * kQ6Stage;
                *reinterpret_cast<unsigned *>(st + 8 * slot + 4 * (i & 1)) = q8.codes;
                const int s4 = __builtin_amdgcn_sdot4((int)q8.codes, 0x01010101, 0, false);
                const int s8 = s4 + dpp_i<kQuadSwap1>(s4);   // the piece's 8 codes
                if ((i & 1) == 0) reinterpret_cast<int *>(st + 288)[slot] = -32 * s8;
                if (i == 0) reinterpret_cast<float *>(st + 256)[j] = q8.d;
            }
            continue;
        }
#pragma unroll
        for (int k = 0; k < PC; ++k) {
            const int m = 2 * k + (lane >> 5);
            if (m < M) {
                uint8_t *st = lds + ((size_t)b * M + m) * kQ6Stage;
                *reinterpret_cast<uint2 *>(st + 8 * sdst) = cv[c][k];
                const int s = __builtin_amdgcn_sdot4((int)cv[c][k].x, 0x01010101, 0, false) +
                              __builtin_amdgcn_sdot4((int)cv[c][k].y, 0x01010101, 0, false);
                reinterpret_cast<int *>(st + 288)[sdst] = -32 * s;
            }
        }
        if ((lane >> 3) < M)
            reinterpret_cast<float *>(lds + ((size_t)b * M + (lane >> 3)) * kQ6Stage + 256)[lane & 7] =
                av[c];
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): this wave's LDS writes done
    __builtin_amdgcn_wave_barrier();

    float acc[V][M];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[v][m] = 0.0f;

    const int slot = (h * 4 + u) * 4;   // the lane's first staged slot (t = 0)
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        if (c >= ncols) break;          // wave-uniform
        const int b = wcol0 + c;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            // bytes into place
            const unsigned odd = qo[v][c];
            const unsigned a0 = __builtin_amdgcn_alignbyte(qa[v][c].y, qa[v][c].x, odd);
            const unsigned a1 = __builtin_amdgcn_alignbyte(qa[v][c].z, qa[v][c].y, odd);
            const unsigned b0 = __builtin_amdgcn_alignbyte(qb[v][c].y, qb[v][c].x, odd);
            const unsigned b1 = __builtin_amdgcn_alignbyte(qb[v][c].z, qb[v][c].y, odd);
            const unsigned h0 = __builtin_amdgcn_alignbyte(qh[v][c].y, qh[v][c].x, odd);
            const unsigned h1 = __builtin_amdgcn_alignbyte(qh[v][c].z, qh[v][c].y, odd);
            const unsigned s0 = __builtin_amdgcn_alignbyte(qs[v][c].y, qs[v][c].x, odd);
            const unsigned s1 = __builtin_amdgcn_alignbyte(qt[v][c], qs[v][c].y, odd);
            const float d = half_lo(qd[v][c]);
            // 6-bit quants of the lane's 8 elements of blocks t = 0..3
            int q[4][2];
            q[0][0] = (int)((a0 & 0x0F0F0F0Fu) | ((h0 << 4) & 0x30303030u));
            q[0][1] = (int)((a1 & 0x0F0F0F0Fu) | ((h1 << 4) & 0x30303030u));
            q[1][0] = (int)((b0 & 0x0F0F0F0Fu) | ((h0 << 2) & 0x30303030u));
            q[1][1] = (int)((b1 & 0x0F0F0F0Fu) | ((h1 << 2) & 0x30303030u));
            q[2][0] = (int)(((a0 >> 4) & 0x0F0F0F0Fu) | (h0 & 0x30303030u));
            q[2][1] = (int)(((a1 >> 4) & 0x0F0F0F0Fu) | (h1 & 0x30303030u));
            q[3][0] = (int)(((b0 >> 4) & 0x0F0F0F0Fu) | ((h0 >> 2) & 0x30303030u));
            q[3][1] = (int)(((b1 >> 4) & 0x0F0F0F0Fu) | ((h1 >> 2) & 0x30303030u));
            // d * sc of the lane's sub-block in each block: sc[8h + 2t + u/2]
            float dsc[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const unsigned word = t < 2 ? s0 : s1;
                const int sc = __builtin_amdgcn_sbfe((int)word, 8 * (2 * (t & 1) + (u >> 1)), 8);
                dsc[t] = d * (float)sc;
            }
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const uint8_t *st = lds + ((size_t)b * M + m) * kQ6Stage;
                const i32x4 c01 = *reinterpret_cast<const i32x4 *>(st + 8 * slot);        // t = 0, 1
                const i32x4 c23 = *reinterpret_cast<const i32x4 *>(st + 8 * slot + 16);   // t = 2, 3
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(st + 256 + 16 * h);
                const i32x4 o4 = *reinterpret_cast<const i32x4 *>(st + 288 + 4 * slot);
                const int cc[4][2] = {{c01.x, c01.y}, {c01.z, c01.w}, {c23.x, c23.y}, {c23.z, c23.w}};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    int p = __builtin_amdgcn_sdot4(q[t][0], cc[t][0], o4[t], false);
                    p = __builtin_amdgcn_sdot4(q[t][1], cc[t][1], p, false);
                    acc[v][m] = fmaf(a4[t], dsc[t] * (float)p, acc[v][m]);
                }
            }
        }
    }

    // ---- the 8 lanes of a row (DPP), then the waves in order (LDS)
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float s = group8_sum(acc[v][m]);
            if ((lane & 7) == 0) red[wave][8 * v + g][m] = s;
        }
    __syncthreads();
    for (int i = threadIdx.x; i < 8 * V * M; i += 64 * nw) {
        const int r = i / M, m = i % M;
        float t = 0.0f;
        for (int k = 0; k < nw; ++k) t += red[k][r][m];
        const int row = row_base + r;
        if (row < N) y[(int64_t)m * N + row] = t;
    }
}

// One product per launch.
template <int M, int CPW, int V, bool FUSED>
__global__ __launch_bounds__(1024) void q6k_gemv_kernel(
    const uint8_t *__restrict__ w, float *__restrict__ y, const int8_t *__restrict__ codes,
    const float *__restrict__ scales, const float *__restrict__ x, int N, int nsb) {
    q6k_rows<M, CPW, V, FUSED>(w, y, codes, scales, x, N, nsb, (int)blockIdx.x * 8 * V);
}

// Products 1.. of a launch of several (product 0 travels in the leading
// kernel arguments, preloaded into registers): weights, fp32 rows (fused
// launches), outputs, rows, first workgroup of each (block0[count] = all).
struct Q6Set {
    const uint8_t *w[kMaxGemvBatch];
    const float *x[kMaxGemvBatch];
    float *y[kMaxGemvBatch];
    int N[kMaxGemvBatch];
    int block0[kMaxGemvBatch + 1];
    int count;
};

// Several products with the same K and M per launch: workgroups are dealt out
// over the products' row blocks in order, each finding its product from its
// block index.  Per row the same work as a one-product launch.
template <int M, int CPW, int V, bool FUSED>
__global__ __launch_bounds__(1024) void q6k_gemv_batch_kernel(
    const uint8_t *w0, float *y0, const float *x0, int N0, int blocks0,
    const int8_t *__restrict__ codes, const float *__restrict__ scales, int nsb, const Q6Set set) {
    if ((int)blockIdx.x < blocks0) {               // uniform
        q6k_rows<M, CPW, V, FUSED>(w0, y0, codes, scales, x0, N0, nsb, (int)blockIdx.x * 8 * V);
        return;
    }
    int pi = 1;
    while (pi + 1 < set.count && (int)blockIdx.x >= set.block0[pi + 1]) ++pi;
    q6k_rows<M, CPW, V, FUSED>(set.w[pi], set.y[pi], codes, scales, set.x[pi], set.N[pi], nsb,
                               ((int)blockIdx.x - set.block0[pi]) * 8 * V);
}

// Activation of a call: prepared Q8 rows (codes, scales) shared by its
// products, or fp32 rows per product (GemvProblem::x).
struct Act {
    const int8_t *codes;
    const float *scales;
    bool fused;
};

template <int M, int CPW, int V>
hipError_t launch_mcv(const GemvProblem *probs, int count, int nsb, const Act &a,
                      hipStream_t stream) {
    const int waves = (nsb + CPW - 1) / CPW;
    const size_t lds = (size_t)nsb * M * kQ6Stage;
    const int rb = 8 * V;
    if (count == 1) {
        const GemvProblem &p = probs[0];
        const int blocks = (int)((p.N + rb - 1) / rb);
        if (a.fused)
            hipLaunchKernelGGL((q6k_gemv_kernel<M, CPW, V, true>), dim3(blocks), dim3(64 * waves),
                               lds, stream, static_cast<const uint8_t *>(p.w), p.y, nullptr,
                               nullptr, p.x, (int)p.N, nsb);
        else
            hipLaunchKernelGGL((q6k_gemv_kernel<M, CPW, V, false>), dim3(blocks), dim3(64 * waves),
                               lds, stream, static_cast<const uint8_t *>(p.w), p.y, a.codes,
                               a.scales, nullptr, (int)p.N, nsb);
        return hipGetLastError();
    }
    Q6Set set = {};
    set.count = count;
    for (int i = 0; i < count; ++i) {
        set.w[i] = static_cast<const uint8_t *>(probs[i].w);
        set.x[i] = probs[i].x;
        set.y[i] = probs[i].y;
        set.N[i] = (int)probs[i].N;
        set.block0[i + 1] = set.block0[i] + (int)((probs[i].N + rb - 1) / rb);
    }
    if (a.fused)
        hipLaunchKernelGGL((q6k_gemv_batch_kernel<M, CPW, V, true>), dim3(set.block0[count]),
                           dim3(64 * waves), lds, stream, set.w[0], set.y[0], set.x[0], set.N[0],
                           set.block0[1], nullptr, nullptr, nsb, set);
    else
        hipLaunchKernelGGL((q6k_gemv_batch_kernel<M, CPW, V, false>), dim3(set.block0[count]),
                           dim3(64 * waves), lds, stream, set.w[0], set.y[0], nullptr, set.N[0],
                           set.block0[1], a.codes, a.scales, nsb, set);
    return hipGetLastError();
}

// Launch shape: columns per wave so that at most 16 waves cover K; rows per
// workgroup (8 V) so that the workgroups (of all the launch's rows) come near
// one or two per CU; at most 4 super-blocks per lane in flight (V * CPW <= 4),
// 2 past M = 4 (registers).  A row's arithmetic does not depend on V.
template <int M>
hipError_t launch_m(const GemvProblem *probs, int count, int nsb, const Act &a,
                    hipStream_t stream) {
    constexpr int kUnits = M <= 4 ? 4 : 2;
    const int cpw = (nsb + kQ6Waves - 1) / kQ6Waves;
    int64_t rows = 0;
    for (int i = 0; i < count; ++i) rows += probs[i].N;
    const int64_t rows_per_cu = (rows + cu_count() - 1) / cu_count();
    const int v = (int)std::max<int64_t>(
        1, std::min<int64_t>(kUnits / cpw, std::max<int64_t>(1, rows_per_cu / 8)));
    if (cpw == 1) {
        if constexpr (kUnits >= 4)
            if (v >= 4) return launch_mcv<M, 1, 4>(probs, count, nsb, a, stream);
        if (v >= 2) return launch_mcv<M, 1, 2>(probs, count, nsb, a, stream);
        return launch_mcv<M, 1, 1>(probs, count, nsb, a, stream);
    }
    if (cpw == 2) {
        if constexpr (kUnits >= 4)
            if (v >= 2) return launch_mcv<M, 2, 2>(probs, count, nsb, a, stream);
        return launch_mcv<M, 2, 1>(probs, count, nsb, a, stream);
    }
    // K of 33..48 super-blocks: 3 columns per wave, one row group
    return launch_mcv<M, 3, 1>(probs, count, nsb, a, stream);
}

hipError_t run_q6k(const GemvProblem *probs, int count, int64_t K, const Act &a, int64_t M,
                   hipStream_t stream) {
    const int nsb = (int)(K / kQK);
    if (!q6k_fits(M, K) || count < 1 || count > kMaxGemvBatch) return hipErrorInvalidValue;
    switch (M) {
    case 1: return launch_m<1>(probs, count, nsb, a, stream);
    case 2: return launch_m<2>(probs, count, nsb, a, stream);
    case 3: return launch_m<3>(probs, count, nsb, a, stream);
    case 4: return launch_m<4>(probs, count, nsb, a, stream);
    case 5: return launch_m<5>(probs, count, nsb, a, stream);
    case 6: return launch_m<6>(probs, count, nsb, a, stream);
    case 7: return launch_m<7>(probs, count, nsb, a, stream);
    case 8: return launch_m<8>(probs, count, nsb, a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

// The staged rows of every column (kQ6Stage bytes per column and row) and the
// cross-wave sums (at most 4 row groups of 8) fit one workgroup's LDS.
bool q6k_fits(int64_t M, int64_t K) {
    if (M < 1 || M > 8 || K < kQK || K % kQK != 0 || K > kQ6MaxK) return false;
    const size_t red = sizeof(float) * kQ6Waves * 8 * 4 * (size_t)M;
    return (size_t)(K / kQK) * (size_t)M * kQ6Stage + red <= lds_limit();
}

hipError_t launch_q6k_gemv(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                           const float *scales, int64_t M, float *y, hipStream_t stream) {
    const GemvProblem p = {w, nullptr, y, N};
    return run_q6k(&p, 1, K, Act{codes, scales, false}, M, stream);
}

hipError_t launch_q6k_quantize_gemv(const uint8_t *w, int64_t N, int64_t K, const float *x,
                                    int64_t M, float *y, hipStream_t stream) {
    const GemvProblem p = {w, x, y, N};
    return run_q6k(&p, 1, K, Act{nullptr, nullptr, true}, M, stream);
}

hipError_t launch_q6k_gemv_batch(const GemvProblem *probs, int count, int64_t K,
                                 const int8_t *codes, const float *scales, int64_t M,
                                 hipStream_t stream) {
    return run_q6k(probs, count, K, Act{codes, scales, false}, M, stream);
}

hipError_t launch_q6k_quantize_gemv_batch(const GemvProblem *probs, int count, int64_t K,
                                          int64_t M, hipStream_t stream) {
    return run_q6k(probs, count, K, Act{nullptr, nullptr, true}, M, stream);
}

}  // namespace q4k
