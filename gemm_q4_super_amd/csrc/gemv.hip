// Decode / small-batch GEMV: y[M][N] = Q8(x)[M][K] * W^T, W in Q4_K, M = 1..8.
//
// Batch-1 decode streams every weight byte once and is bound by memory
// bandwidth ("genie-ai-runtime ...", section 2, the decode ceiling), so this
// kernel is built around the HBM stream and uses no matrix cores:
//
//  * Lane <-> 16-byte quant chunk.  A super-block is 144 B = a 16-B header
//    plus eight 16-B quant chunks; 8 lanes (a "group") take one super-block,
//    lane l loading chunk l with one 16-B load and the header with another.
//    (The pages' Path C reads four packed quant bytes as one 32-bit load; on
//    gfx950 a lane moves 16 B per load.)
//  * Sub-block integer dots with v_dot4 (sdot4); the partner lanes of a chunk
//    pair exchange one half with a DPP quad swap, after which lane l holds the
//    exact int32 dot of sub-block j = l and applies its fp32 epilogue
//    acc += a_j * (d*sc_j*D_j - dmin*mn_j*S_j)   (helpers in q4k_device.h).
//  * Workgroup = W waves splitting the K/256 super-block columns of the same
//    8*T rows; group g of every wave owns rows 8t+g.  A wave issues the loads
//    of all its columns (up to CPW) before any arithmetic, so one DRAM round
//    trip covers them.  The activation chunk of a column is reused over the T
//    row tiles and all 8 groups.  Per-lane sums reduce over the 8 lanes by
//    DPP, then over the W waves through LDS in a fixed order (deterministic).
//  * Fused variant (q4k_quantize_gemv): the activation arrives as fp32 and
//    each wave quantizes the Q8 blocks of its own columns into LDS (same
//    arithmetic as q4k_quantize_act, so the codes are bit-identical) while its
//    weight loads are in flight -- one launch instead of two per call.
#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kMaxWaves = 16;
constexpr int kMaxPieces = 16;

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp_f<kQuadSwap1>(v));
    v = fmaxf(v, dpp_f<kQuadSwap2>(v));
    v = fmaxf(v, dpp_f<kRowHalfMirror>(v));
    return v;
}
__device__ __forceinline__ int group8_isum(int v) {
    v += dpp_i<kQuadSwap1>(v);
    v += dpp_i<kQuadSwap2>(v);
    v += dpp_i<kRowHalfMirror>(v);
    return v;
}
// Branch-free: an all-zero block (d == 0) divides by 1 and selects 0.
__device__ __forceinline__ int quant1(float x, float d) {
    const bool zero = d == 0.0f;
    float r = __builtin_rintf(x / (zero ? 1.0f : d));
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return zero ? 0 : (int)r;
}

// Per-wave LDS of the fused variant: Q8 of the wave's CPW columns, M rows.
template <int M, int CPW>
struct WaveQ8 {
    int8_t c[M][CPW][256];
    float a[M][CPW][8];
    float s[M][CPW][8];
};

// Kernel arguments.  The fused variant takes up to kMaxPieces row ranges
// ("pieces") of one or more products with the same K and M: piece p covers
// rows [0, N[p]) of the matrix at w[p] and writes y[p][m * ldy[p] + row]; the
// host cuts large products into pieces of similar size, so that blockIdx.y
// names the piece and workgroups past a short piece's rows exit at once.  The
// other variant multiplies prepared Q8 rows by one matrix.  Every value a
// workgroup needs is addressed from blockIdx alone: one round of scalar loads.
template <bool FUSED> struct GemvArgs;
template <> struct GemvArgs<true> {
    const uint8_t *w[kMaxPieces];
    const float *x[kMaxPieces];
    float *y[kMaxPieces];
    int N[kMaxPieces];
    int ldy[kMaxPieces];
};
template <> struct GemvArgs<false> {
    const uint8_t *w[1];
    float *y[1];
    int N[1];
    int ldy[1];
    const int8_t *codes;
    const float *scales;
    const int32_t *sums;
};

template <int M, int T, int CPW, bool FUSED>
__global__ __launch_bounds__(1024) void gemv_kernel(const GemvArgs<FUSED> B, int nsb) {
    __shared__ float red[kMaxWaves][8 * T][M];
    extern __shared__ __attribute__((aligned(16))) uint8_t dyn[];

    const int p = FUSED ? (int)blockIdx.y : 0;
    const uint8_t *__restrict__ w = B.w[p];
    float *__restrict__ y = B.y[p];
    const int N = B.N[p];
    const int ldy = B.ldy[p];
    const float *__restrict__ x = nullptr;
    const int8_t *__restrict__ codes = nullptr;
    const float *__restrict__ scales = nullptr;
    const int32_t *__restrict__ sums = nullptr;
    if constexpr (FUSED) {
        x = B.x[p];
        asm volatile("" ::"s"(w), "s"(x), "s"(y), "s"(N), "s"(ldy), "s"(nsb));
    } else {
        codes = B.codes;
        scales = B.scales;
        sums = B.sums;
        asm volatile("" ::"s"(w), "s"(codes), "s"(scales), "s"(sums), "s"(y), "s"(N), "s"(nsb));
    }
    const int wg = (int)blockIdx.x;
    if (wg * (8 * T) >= N) return;   // past this piece's rows (whole workgroup)

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // the launch's wave count, from the kernel arguments (as the host sizes it)
    const int nwaves = (nsb + CPW - 1) / CPW < kMaxWaves ? (nsb + CPW - 1) / CPW : kMaxWaves;
    const int grp = lane >> 3;     // row within a tile of 8
    const LaneMap L(lane & 7);     // chunk index == sub-block owned after the swap
    const int K = nsb * 256;
    const int nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * 144;
    const int row0 = wg * (8 * T);
    WaveQ8<M, CPW> *q8 = reinterpret_cast<WaveQ8<M, CPW> *>(dyn) + wave;

    float acc[T][M];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[t][m] = 0.0f;

    // Columns [b0, b0 + CPW) of this wave; a wave with more than CPW columns
    // (K beyond 16 * CPW super-blocks) takes them in groups of CPW.
    // Activation loads go out before the weight loads: the load counter
    // retires in order, so data wanted first must be requested first (the
    // quantization, or column 0's dots, then overlaps the weight stream).
    constexpr bool kActFirst = FUSED || M * CPW * T <= 6;
    for (int b0 = wave * CPW; b0 < nsb; b0 += nwaves * CPW) {
        f32x4 xv[FUSED ? M : 1][FUSED ? CPW : 1];
        i32x4 pA[kActFirst && !FUSED ? CPW : 1][M], pB[kActFirst && !FUSED ? CPW : 1][M];
        float pa[kActFirst && !FUSED ? CPW : 1][M];
        int ps[kActFirst && !FUSED ? CPW : 1][M];   // converted at use, after the loads
        if constexpr (FUSED) {
            const int blk = lane >> 3, sub = lane & 7;
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    // clamped, branch-free: columns past nsb are never used
                    const int b = min(b0 + c, nsb - 1);
                    xv[m][c] = *reinterpret_cast<const f32x4 *>(x + (int64_t)m * K + 256 * b +
                                                                32 * blk + 4 * sub);
                }
        } else if constexpr (kActFirst) {
#pragma unroll
            for (int c = 0; c < CPW; ++c)
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const int b = min(b0 + c, nsb - 1);   // clamped: unused past nsb
                    const int8_t *cm = codes + (int64_t)m * K + 256 * b;
                    pA[c][m] = *reinterpret_cast<const i32x4 *>(cm + L.offA);
                    pB[c][m] = *reinterpret_cast<const i32x4 *>(cm + L.offB);
                    pa[c][m] = scales[(int64_t)m * nblk + 8 * b + L.l];
                    ps[c][m] = sums[(int64_t)m * nblk + 8 * b + L.l];
                }
        }
        __builtin_amdgcn_sched_barrier(0);   // activation loads stay first
        // Branch-free weight loads from clamped addresses: a load under a
        // branch makes the compiler wait for every load at the join, which
        // would serialize the activation work behind the weight stream.  Rows
        // past N compute on row N-1 and are never written; columns past nsb
        // are skipped below.
        u32x4 hd[CPW][T], qw[CPW][T];
#pragma unroll
        for (int c = 0; c < CPW; ++c)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                const int row = row0 + 8 * t + grp, b = b0 + c;
                const uint8_t *sb = w + (int64_t)min(row, N - 1) * row_bytes +
                                    (int64_t)min(b, nsb - 1) * 144;
                hd[c][t] = load_stream16(sb);
                qw[c][t] = load_stream16(sb + 16 + 16 * L.l);
            }
        // Keep every load of the group ahead of the arithmetic below.
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (FUSED) {
            // Quantize this wave's columns: lane -> block lane/8 of the column,
            // 4 values at 4*(lane%8) within the block.
            const int blk = lane >> 3, sub = lane & 7;
#pragma unroll
            for (int m = 0; m < M; ++m)
#pragma unroll
                for (int c = 0; c < CPW; ++c) {
                    const f32x4 v = xv[m][c];
                    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])),
                                       fmaxf(fabsf(v[2]), fabsf(v[3])));
                    amax = group8_max(amax);
                    const float d = amax / 127.0f;
                    const int c0 = quant1(v[0], d), c1 = quant1(v[1], d);
                    const int c2 = quant1(v[2], d), c3 = quant1(v[3], d);
                    *reinterpret_cast<int *>(&q8->c[m][c][32 * blk + 4 * sub]) =
                        (c0 & 0xFF) | ((c1 & 0xFF) << 8) | ((c2 & 0xFF) << 16) |
                        (int)((unsigned)c3 << 24);
                    const int ssum = group8_isum(c0 + c1 + c2 + c3);
                    if (sub == 0) {
                        q8->a[m][c][blk] = d;
                        q8->s[m][c][blk] = (float)ssum;
                    }
                }
            // LDS written and read by this wave only: wait for the writes.
            __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
            __builtin_amdgcn_wave_barrier();
        }
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const int b = b0 + c;
            if (b >= nsb) break;                 // wave-uniform
            // Activation chunk of this column, reused over the row tiles.
            i32x4 cA[M], cB[M];
            float a[M];
            float s[M];
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if constexpr (FUSED) {
                    cA[m] = *reinterpret_cast<const i32x4 *>(&q8->c[m][c][L.offA]);
                    cB[m] = *reinterpret_cast<const i32x4 *>(&q8->c[m][c][L.offB]);
                    a[m] = q8->a[m][c][L.l];
                    s[m] = q8->s[m][c][L.l];
                } else if constexpr (kActFirst) {
                    cA[m] = pA[c][m];
                    cB[m] = pB[c][m];
                    a[m] = pa[c][m];
                    s[m] = (float)ps[c][m];
                } else {
                    const int8_t *cm = codes + (int64_t)m * K + 256 * b;
                    cA[m] = *reinterpret_cast<const i32x4 *>(cm + L.offA);
                    cB[m] = *reinterpret_cast<const i32x4 *>(cm + L.offB);
                    a[m] = scales[(int64_t)m * nblk + 8 * b + L.l];
                    s[m] = (float)sums[(int64_t)m * nblk + 8 * b + L.l];
                }
            }
#pragma unroll
            for (int t = 0; t < T; ++t) {
                float ds, dm;
                decode_scale(L, hd[c][t], ds, dm);
                int qlo[4], qhi[4];
                unpack_nibbles(qw[c][t], qlo, qhi);
#pragma unroll
                for (int m = 0; m < M; ++m) {
                    const int D = subblock_dot(L, qlo, qhi, cA[m], cB[m]);
                    acc[t][m] = fmaf(a[m], fmaf(ds, (float)D, -(dm * s[m])), acc[t][m]);
                }
            }
        }
        if constexpr (FUSED) __builtin_amdgcn_wave_barrier();   // LDS reuse by the next group
    }

    // Reduce the 8 sub-block lanes of each group, then the waves via LDS.
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const float v = group8_sum(acc[t][m]);
            if (L.l == 0) red[wave][8 * t + grp][m] = v;
        }
    __syncthreads();
    for (int i = threadIdx.x; i < 8 * T * M; i += 64 * nwaves) {
        const int r = i / M, m = i % M;
        float v = 0.0f;
        for (int wv = 0; wv < nwaves; ++wv) v += red[wv][r][m];
        const int row = row0 + r;
        if (row < N) y[(int64_t)m * ldy + row] = v;
    }
}

template <int M, int T, int CPW, bool FUSED>
hipError_t launch_mtc(const GemvArgs<FUSED> &B, int pieces, int nsb, hipStream_t stream) {
    const int nwaves = (nsb + CPW - 1) / CPW < kMaxWaves ? (nsb + CPW - 1) / CPW : kMaxWaves;
    const int rows_per_wg = 8 * T;
    int tiles = 0;
    for (int i = 0; i < pieces; ++i) {
        const int t = (B.N[i] + rows_per_wg - 1) / rows_per_wg;
        tiles = t > tiles ? t : tiles;
    }
    const size_t lds = FUSED ? sizeof(WaveQ8<M, CPW>) * nwaves : 0;
    hipLaunchKernelGGL((gemv_kernel<M, T, CPW, FUSED>), dim3(tiles, pieces),
                       dim3(64 * nwaves), lds, stream, B, nsb);
    return hipGetLastError();
}

// One call's products as the host received them.
struct Req {
    const GemvProblem *probs;   // fused: `count` products
    int count;
    const uint8_t *w;           // plain: one matrix and its Q8 rows
    float *y;
    int N;
    const int8_t *codes;
    const float *scales;
    const int32_t *sums;
    int64_t rows;               // sum of the products' N
};

// Cut the products into pieces of at most C rows, C being one of the
// products' own row counts (rounded up to whole workgroups): the choice that
// launches the fewest workgroups (grid = pieces x tiles of C) with at most
// kMaxPieces pieces.  E.g. N = {4096, 1024, 1024} becomes six pieces of 1024.
int build_args(const Req &r, int rows_per_wg, int nsb, GemvArgs<true> &B) {
    auto tiles = [&](int64_t n) { return (n + rows_per_wg - 1) / rows_per_wg; };
    int64_t C = 0, best = -1;
    for (int c = 0; c < r.count; ++c) {
        const int64_t cand = tiles(r.probs[c].N) * rows_per_wg;
        int64_t pieces = 0;
        for (int i = 0; i < r.count; ++i) pieces += (r.probs[i].N + cand - 1) / cand;
        const int64_t cost = pieces * (cand / rows_per_wg);
        if (pieces <= kMaxPieces && (best < 0 || cost < best || (cost == best && cand > C))) {
            best = cost;
            C = cand;
        }
    }
    const int64_t row_bytes = (int64_t)nsb * 144;
    int n = 0;
    for (int i = 0; i < r.count; ++i) {
        const GemvProblem &q = r.probs[i];
        for (int64_t r0 = 0; r0 < q.N; r0 += C, ++n) {
            B.w[n] = static_cast<const uint8_t *>(q.w) + r0 * row_bytes;
            B.x[n] = q.x;
            B.y[n] = q.y + r0;
            B.N[n] = (int)(q.N - r0 < C ? q.N - r0 : C);
            B.ldy[n] = (int)q.N;
        }
    }
    return n;
}

int build_args(const Req &r, int, int, GemvArgs<false> &B) {
    B.w[0] = r.w;
    B.y[0] = r.y;
    B.N[0] = r.N;
    B.ldy[0] = r.N;
    B.codes = r.codes;
    B.scales = r.scales;
    B.sums = r.sums;
    return 1;
}

template <int M, int T, int CPW, bool FUSED>
hipError_t go(const Req &r, int nsb, hipStream_t stream) {
    GemvArgs<FUSED> B = {};
    const int pieces = build_args(r, 8 * T, nsb, B);
    return launch_mtc<M, T, CPW, FUSED>(B, pieces, nsb, stream);
}

template <int M, bool FUSED>
hipError_t launch_m(const Req &r, int nsb, hipStream_t stream) {
    // Columns per wave: as few as the 16-wave workgroup allows; two row tiles
    // per workgroup once the launch has enough rows to fill the chip.
    if constexpr (M <= 2) {
        if (r.rows >= 4096) {
            if (nsb <= 16) return go<M, 2, 1, FUSED>(r, nsb, stream);
            if (nsb <= 32) return go<M, 2, 2, FUSED>(r, nsb, stream);
            return go<M, 2, 3, FUSED>(r, nsb, stream);
        }
    }
    if (nsb <= 16) return go<M, 1, 1, FUSED>(r, nsb, stream);
    if (nsb <= 32) return go<M, 1, 2, FUSED>(r, nsb, stream);
    return go<M, 1, 3, FUSED>(r, nsb, stream);
}

template <bool FUSED>
hipError_t dispatch(const Req &r, int64_t K, int64_t M, hipStream_t stream) {
    const int nsb = (int)(K / kQK);
    switch (M) {
    case 1: return launch_m<1, FUSED>(r, nsb, stream);
    case 2: return launch_m<2, FUSED>(r, nsb, stream);
    case 3: return launch_m<3, FUSED>(r, nsb, stream);
    case 4: return launch_m<4, FUSED>(r, nsb, stream);
    case 5: return launch_m<5, FUSED>(r, nsb, stream);
    case 6: return launch_m<6, FUSED>(r, nsb, stream);
    case 7: return launch_m<7, FUSED>(r, nsb, stream);
    case 8: return launch_m<8, FUSED>(r, nsb, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_gemv(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       hipStream_t stream) {
    Req r = {};
    r.w = w;
    r.y = y;
    r.N = (int)N;
    r.codes = codes;
    r.scales = scales;
    r.sums = sums;
    r.rows = N;
    return dispatch<false>(r, K, M, stream);
}

hipError_t launch_quantize_gemv_batch(const GemvProblem *probs, int count, int64_t K,
                                      int64_t M, hipStream_t stream) {
    Req r = {};
    r.probs = probs;
    r.count = count;
    for (int i = 0; i < count; ++i) r.rows += probs[i].N;
    return dispatch<true>(r, K, M, stream);
}

hipError_t launch_quantize_gemv(const uint8_t *w, int64_t N, int64_t K, const float *x,
                                int64_t M, float *y, hipStream_t stream) {
    const GemvProblem p = {w, x, y, N};
    return launch_quantize_gemv_batch(&p, 1, K, M, stream);
}

}  // namespace q4k
