// Streaming Q4_K x Q8 GEMV for decode and small batches (M = 1..8 activation
// rows whose Q8 form fits one workgroup's LDS, e.g. M = 8 at K = 9728 in the
// 160 KB of a gfx950 workgroup): y_i = Q8(x_i) * W_i^T for up to 8 products with the
// same K and M in one launch.  Included by qgemv.hip (fp32 activations,
// quantized inside the kernel) and gemv.hip (prepared Q8 rows); both run the
// same kernel body and the same partition, so they are bit-identical.
//
// Batch-1 decode streams every weight byte once and is bound by memory
// bandwidth ("genie-ai-runtime ...", section 2, the decode ceiling).  At
// 2-30 MB per launch what keeps a kernel from that ceiling is latency and
// balance: every CU should hold the same number of weight bytes, all of them
// requested before any arithmetic waits.  So:
//
//  * Lane <-> 16-byte quant chunk: 8 lanes (a "group") take one 144-byte
//    super-block, lane l loading quant chunk l and one dword of the 16-byte
//    header (spread over the lane quad by DPP); integer
//    sub-block dots by sdot4 with a DPP quad swap, fp32 epilogue
//    acc += a_j * (d*sc_j*D_j - dmin*mn_j*S_j)  (helpers in q4k_device.h).
//  * Layout of a wave's 8 groups: RG rows x S = 8/RG column slots (RG = 8,
//    4 or 2); each slot owns CPW consecutive super-block columns, so a wave
//    covers RG rows and S*CPW columns, and a workgroup of W waves all K/256
//    columns.  A lane holds V row groups: a workgroup's block is RB = RG*V
//    rows.  The host picks (RG, V, CPW) per launch so that workgroups hold
//    equal row blocks and are spread evenly over the CUs (e.g. 2560 rows on
//    256 CUs: RG = 2, V = 5, one 10-row block per CU).
//  * Every wave issues the loads of all its V*CPW super-blocks before any
//    arithmetic: the workgroup's whole block is in flight at once.
//  * Activation: each wave stages the Q8 rows of its own S*CPW columns in LDS
//    (quantizing fp32 x with the quantizer q4k_quantize_act uses,
//    quantize_block8, so the codes are bit-identical, or copying prepared
//    codes) and reads only those, so no workgroup barrier waits for the
//    staging.  The activation loads go out before the weight loads (the load
//    counter retires in order); waves whose weight loads would queue behind
//    other waves' (past the first four of a wide workgroup) quantize before
//    issuing them.
//  * Each super-block's term is summed over its 8 lanes by DPP and parked in
//    LDS; a row then adds its K/256 terms in column order.  That order does
//    not depend on (RG, V, CPW), so single, batched, fused and prepared calls
//    give the same bits whatever shape the host picks.
//  * Products are cut on the host into row "pieces" of similar size; the
//    piece is blockIdx.y and the first piece's arguments come first in the
//    argument block (preloaded into registers), so a workgroup needs at most
//    one round of scalar loads before it issues its weight loads.
#pragma once

#include <atomic>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace stream {

constexpr int kWaves = 16;     // waves per workgroup, at most
constexpr int kPieces = 16;    // row pieces per launch, at most

// Pieces 1.. of a launch (piece 0 travels in the leading kernel arguments).
struct Pieces {
    const uint8_t *w[kPieces];
    const float *x[kPieces];
    float *y[kPieces];
    const float *r[kPieces];   // residual added to the piece's output, or null
    int N[kPieces];      // rows of the piece
    int ldy[kPieces];    // row stride of y (the product's N)
};

// Per-call inputs beside the products: the prepared Q8 rows of the plain
// GEMV (null when the kernel quantizes), and a residual [M][N] added to the
// output of a single product in the last step (null for none).
struct Prepared {
    const int8_t *codes;
    const float *scales;
    const int32_t *sums;
    const float *residual = nullptr;
};

// Launch shape, packed into one kernel argument: lg(RG) in bits 0-1,
// V in bits 2-5, W (waves) in bits 6-10.
__host__ __device__ constexpr int pack_cfg(int lg_rg, int v, int waves) {
    return lg_rg | (v << 2) | (waves << 6);
}

// Up to this many super-blocks per lane (V * CPW), by activation rows.
template <int M>
constexpr int max_units() {
    return M <= 2 ? 8 : M <= 4 ? 4 : M <= 6 ? 2 : 1;
}

// LDS of the staged Q8 activation, every column: codes, scales, sums.
__host__ __device__ constexpr size_t q8_bytes(int M, int nsb) {
    return (size_t)M * nsb * (256 + 32 + 32);
}
// LDS of the per-super-block terms of a workgroup's block of rows.
__host__ __device__ constexpr size_t col_bytes(int M, int RB, int nsb) {
    return sizeof(float) * (size_t)RB * nsb * M;
}

// Activation staging columns per wave held in registers at once.
template <int M>
constexpr int stage_batch() {
    return M <= 1 ? 4 : M <= 2 ? 2 : 1;
}

template <int M, int CPW, int V, bool FUSED, bool RES>
__global__ __launch_bounds__(1024) void stream_gemv_kernel(
    const uint8_t *__restrict__ w0, const float *__restrict__ x0, float *y0, const float *r0,
    int N0, int ldy0, int nsb, int cfg, const Pieces P, const Prepared Q) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

    // Piece of this workgroup: piece 0 from the leading arguments, others
    // from the argument block.
    const int p = (int)blockIdx.y;
    const uint8_t *__restrict__ w = w0;
    const float *__restrict__ x = x0;
    // y and res may be the same buffer (an in-place residual add): each
    // output element is read and then written by one thread.  RES: the call
    // has a residual (res is not null).
    float *y = y0;
    const float *res = r0;
    int N = N0, ldy = ldy0;
    if (p != 0) {
        w = P.w[p];
        x = P.x[p];
        y = P.y[p];
        res = P.r[p];
        N = P.N[p];
        ldy = P.ldy[p];
    }
    const int lg_rg = cfg & 3, RG = 1 << lg_rg;
    const int nw = (cfg >> 6) & 31;
    const int RB = RG * V;
    const int row_base = (int)blockIdx.x * RB;
    if (row_base >= N) return;   // whole workgroup: past this piece's rows

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 3;                 // group
    const int r = g & (RG - 1);              // row within an RG-row set
    const int s = g >> lg_rg;                // column slot
    const int S = 8 >> lg_rg;
    const LaneMap L(lane & 7);
    const ScaleBits SB(lane & 7);
    const int K = nsb * 256;
    const int nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * 144;
    const int wcol0 = wave * S * CPW;        // the wave's columns: [wcol0, wcol0 + S*CPW)
    const int col0 = wcol0 + s * CPW;        // this lane's first column

    int8_t *qc = reinterpret_cast<int8_t *>(lds);                       // [M][nsb][256]
    float *qa = reinterpret_cast<float *>(lds + (size_t)M * nsb * 256);  // [M][nsb][8]
    float *qs = qa + (size_t)M * nblk;                                   // [M][nsb][8]
    float *colsum = reinterpret_cast<float *>(lds + q8_bytes(M, nsb));    // [RB][nsb][M]

    // ---- activation loads (first batch of staged columns), then weights
    constexpr int QB = stage_batch<M>();
    const int blk = lane >> 3, sub = lane & 7;
    const int ncols = min(S * CPW, nsb - wcol0);   // the wave's live columns (>= 1)
    f32x4 xv[QB][M];
    int pc[QB][M];
    float psc[QB][M];
    int psu[QB][M];
    auto stage_load = [&](int j0) {
#pragma unroll
        for (int j = 0; j < QB; ++j) {
            // Wave-uniform guard: these loads precede every weight load, so the
            // waits for them stay exact.
            if (j0 + j >= ncols) break;
            const int b = wcol0 + j0 + j;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                if constexpr (FUSED) {
                    xv[j][m] = *reinterpret_cast<const f32x4 *>(x + (int64_t)m * K + 256 * b +
                                                                32 * blk + 4 * sub);
                } else {
                    pc[j][m] = *reinterpret_cast<const int *>(Q.codes + (int64_t)m * K +
                                                              256 * b + 4 * lane);
                    psc[j][m] = Q.scales[(int64_t)m * nblk + 8 * b + sub];
                    psu[j][m] = Q.sums[(int64_t)m * nblk + 8 * b + sub];
                }
            }
        }
    };
    auto stage_store = [&](int j0) {
#pragma unroll
        for (int j = 0; j < QB; ++j) {
            if (j0 + j >= ncols) break;   // wave-uniform
            const int b = wcol0 + j0 + j;
#pragma unroll
            for (int m = 0; m < M; ++m) {
                int8_t *cm = qc + ((size_t)m * nsb + b) * 256;
                float *am = qa + ((size_t)m * nsb + b) * 8;
                float *sm = qs + ((size_t)m * nsb + b) * 8;
                if constexpr (FUSED) {
                    // lane -> block lane/8 of the column, 4 values at 4*(lane%8)
                    const Q8Lane qb = quantize_block8(xv[j][m]);
                    *reinterpret_cast<unsigned *>(cm + 32 * blk + 4 * sub) = qb.codes;
                    if (sub == 0) {
                        am[blk] = qb.d;
                        sm[blk] = (float)qb.sum;
                    }
                } else {
                    *reinterpret_cast<int *>(cm + 4 * lane) = pc[j][m];
                    if (lane < 8) {
                        am[lane] = psc[j][m];
                        sm[lane] = (float)psu[j][m];
                    }
                }
            }
        }
    };
    stage_load(0);
    // In a workgroup of 8 or more waves, the loads of waves past the first four
    // queue behind the first four's data (a CU holds about four waves' loads in
    // flight), so those waves quantize their columns first: the quantization
    // then no longer sits between their weights' arrival and the dots.
    const bool stage_first = nw >= 8 && wave >= 4;   // wave-uniform
    auto stage_all = [&]() {
        stage_store(0);
        for (int j0 = QB; j0 < ncols; j0 += QB) {   // more columns than one batch
            stage_load(j0);
            stage_store(j0);
        }
    };
    if (stage_first) stage_all();
    __builtin_amdgcn_sched_barrier(0);

    // Branch-free weight loads from clamped addresses (a load under a branch
    // makes the compiler wait for every load at the join).  Rows past N read
    // row N-1 and are never written; columns past nsb are never added.
    // The 16-byte header of a super-block is read as four dwords, one per lane
    // of each lane quad (lane l: dword l % 4), and spread over the quad by DPP
    // at use: a quarter of the address work of a 16-byte load per lane.
    // Addresses: the workgroup's first row in 64 bits (scalar), then 32-bit
    // offsets within its block of rows (at most 64 rows of 18 KB).
    const uint8_t *__restrict__ wb = w + (int64_t)row_base * row_bytes;
    const unsigned hoff = 4u * (lane & 3), qoff = 16u + 16u * L.l;
    unsigned hd[V][CPW];
    u32x4 qw[V][CPW];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int c = 0; c < CPW; ++c) {
            const unsigned rr = (unsigned)(min(row_base + v * RG + r, N - 1) - row_base);
            const unsigned b = (unsigned)min(col0 + c, nsb - 1);
            const unsigned off = __umul24(rr, (unsigned)row_bytes) + b * 144u;
            hd[v][c] = *reinterpret_cast<const unsigned *>(wb + (off + hoff));
            qw[v][c] = load_weights16(wb + (off + qoff));
        }
    // The residual element of this thread's first output in the last step,
    // requested behind the weights (loads complete in order, so it delays no
    // earlier wait) and long before its use.  A compile-time switch, not a
    // branch: a load under a branch leaves the compiler's count of loads in
    // flight ambiguous, and the waits for the activation would then also wait
    // for a weight.  The address is clamped into the piece (the value is used
    // only if in range).
    float res_first = 0.0f;
    if constexpr (RES) {
        const int i = min((int)threadIdx.x, RB * M - 1);
        const int row = min(row_base + i / M, N - 1);
        res_first = res[(int64_t)(i % M) * ldy + row];
    }
    __builtin_amdgcn_sched_barrier(0);

    if (!stage_first) stage_all();
    // LDS written and read by this wave only: wait for its writes.
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();

    // ---- dots: column c outer (its activation read once), row group v inner.
    // Each super-block's term is summed over its 8 lanes and parked in LDS.
#pragma unroll
    for (int c = 0; c < CPW; ++c) {
        const int b = col0 + c;
        const bool live = b < nsb;               // per group (slots differ)
        const int bc = min(b, nsb - 1);
        float *cs = colsum + ((size_t)r * nsb + bc) * M;   // row group v adds v*RG*nsb*M
        i32x4 cA[M], cB[M];
        float a[M], sm[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int8_t *cm = qc + ((size_t)m * nsb + bc) * 256;
            cA[m] = *reinterpret_cast<const i32x4 *>(cm + L.offA);
            cB[m] = *reinterpret_cast<const i32x4 *>(cm + L.offB);
            a[m] = qa[((size_t)m * nsb + bc) * 8 + L.l];
            sm[m] = qs[((size_t)m * nsb + bc) * 8 + L.l];
        }
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float ds, dm;
            decode_scale_bits(SB, quad_gather(hd[v][c]), ds, dm);
            int qlo[4], qhi[4];
            unpack_nibbles(qw[v][c], qlo, qhi);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int D = subblock_dot(L, qlo, qhi, cA[m], cB[m]);
                const float t = superblock_term(a[m], subblock_factor(ds, D, dm, sm[m]));
                if (L.l == 0 && live) cs[v * RG * nsb * M + m] = t;
            }
        }
    }
    __syncthreads();

    // ---- a row adds its column terms in column order: the same order for any
    // (RG, V, CPW), so every launch shape gives the same bits.  A residual is
    // added to the finished sum, one fp32 rounding.
    for (int i = threadIdx.x; i < RB * M; i += 64 * nw) {
        const int rr = i / M, m = i % M;          // row of the block
        const float *cs = colsum + (size_t)rr * nsb * M + m;
        float t = 0.0f;
        for (int b = 0; b < nsb; ++b) t += cs[(size_t)b * M];
        const int row = row_base + rr;
        if (row < N) {
            const int64_t o = (int64_t)m * ldy + row;
            if constexpr (RES) t += i == (int)threadIdx.x ? res_first : res[o];
            y[o] = t;
        }
    }
}

// ------------------------------------------------------------------- host --


struct Plan {
    int lg_rg = 3, v = 1, cpw = 1, waves = 1;
    int64_t C = 0;          // rows per piece
    double cost = 0;
    bool ok = false;
};

// Rows per piece: one of the products' own row counts rounded up to whole
// blocks (so pieces come out of similar size), with at most kPieces pieces.
// Cost, in rows of weights: the workgroups the busiest CU receives (the
// dispatcher deals them out evenly) times what each costs: its block of rows,
// scaled up by the share of lanes without a live column and by 2% per wave of
// the workgroup (each wave pays the staging, barriers and sums), plus the
// activation it stages (about 2 rows' worth per fp32 activation row, 0.6 for
// prepared int8 codes).  Ties go to fewer rows per wave instruction, then
// fewer columns and row groups per lane.  Fitted to a sweep of every launch
// shape over the decode projections on MI355X (best: 2560 x 4096 and
// 2560 x 9728: RG 2, V 5; 6144 and 2 x 9728 rows at K = 2560: RG 4, V 2 and
// V 4 or 5).
inline void consider(Plan &best, const GemvProblem *probs, int count, int nsb, int M, bool fused,
                     int lg_rg, int v, int cpw) {
    const int RG = 1 << lg_rg, S = 8 >> lg_rg, RB = RG * v;
    const int waves = (nsb + S * cpw - 1) / (S * cpw);
    if (waves > kWaves) return;
    const size_t lds = q8_bytes(M, nsb) + col_bytes(M, RB, nsb);
    if (lds > lds_limit()) return;
    const int cus = cu_count();
    for (int c = 0; c < count; ++c) {
        const int64_t C = (probs[c].N + RB - 1) / RB * RB;
        int64_t pieces = 0, wgs = 0;
        for (int i = 0; i < count; ++i) {
            pieces += (probs[i].N + C - 1) / C;
            wgs += (probs[i].N + RB - 1) / RB;   // the last piece of each may be short
        }
        if (pieces > kPieces) continue;
        const int64_t per = (wgs + cus - 1) / cus;
        const double eff = (double)nsb / ((double)waves * S * cpw);
        const double cost = (double)per * (RB / eff * (1.0 + 0.02 * waves) + (fused ? 2.0 : 0.6) * M) +
                            1e-6 * (double)(pieces * ((C / RB) - 1));
        if (!best.ok || cost < best.cost - 1e-9) {
            best.ok = true;
            best.cost = cost;
            best.lg_rg = lg_rg;
            best.v = v;
            best.cpw = cpw;
            best.waves = waves;
            best.C = C;
        }
    }
}

template <int M, int CPW, int V, bool FUSED, bool RES>
hipError_t launch_plan(const Plan &pl, const GemvProblem *probs, int count, int nsb,
                       const Prepared &Q, hipStream_t stream) {
    const int RB = (1 << pl.lg_rg) * V;
    const size_t lds = q8_bytes(M, nsb) + col_bytes(M, RB, nsb);
    // pieces
    const uint8_t *w[kPieces];
    const float *x[kPieces];
    float *y[kPieces];
    const float *r[kPieces];
    int N[kPieces], ldy[kPieces];
    const int64_t row_bytes = (int64_t)nsb * 144;
    int n = 0;
    for (int i = 0; i < count; ++i) {
        const GemvProblem &q = probs[i];
        for (int64_t r0 = 0; r0 < q.N; r0 += pl.C, ++n) {
            w[n] = static_cast<const uint8_t *>(q.w) + r0 * row_bytes;
            x[n] = q.x;
            y[n] = q.y + r0;
            r[n] = Q.residual ? Q.residual + r0 : nullptr;
            N[n] = (int)(q.N - r0 < pl.C ? q.N - r0 : pl.C);
            ldy[n] = (int)q.N;
        }
    }
    Pieces P = {};
    for (int i = 1; i < n; ++i) {
        P.w[i] = w[i];
        P.x[i] = x[i];
        P.y[i] = y[i];
        P.r[i] = r[i];
        P.N[i] = N[i];
        P.ldy[i] = ldy[i];
    }
    const int gx = (int)((pl.C + RB - 1) / RB);
    hipLaunchKernelGGL((stream_gemv_kernel<M, CPW, V, FUSED, RES>), dim3(gx, n), dim3(64 * pl.waves),
                       lds, stream, w[0], x[0], y[0], r[0], N[0], ldy[0], nsb,
                       pack_cfg(pl.lg_rg, V, pl.waves), P, Q);
    return hipGetLastError();
}

// Instances: V * CPW <= max_units<M>().
template <int M, bool FUSED, bool RES>
struct Table {
    static constexpr int U = max_units<M>();
    template <int CPW, int V>
    static void add(Plan &best, const GemvProblem *probs, int count, int nsb, int lg_rg) {
        if constexpr (V * CPW <= U) consider(best, probs, count, nsb, M, FUSED, lg_rg, V, CPW);
    }
    template <int CPW>
    static void add_v(Plan &best, const GemvProblem *probs, int count, int nsb, int lg_rg) {
        add<CPW, 1>(best, probs, count, nsb, lg_rg);
        add<CPW, 2>(best, probs, count, nsb, lg_rg);
        add<CPW, 3>(best, probs, count, nsb, lg_rg);
        add<CPW, 4>(best, probs, count, nsb, lg_rg);
        add<CPW, 5>(best, probs, count, nsb, lg_rg);
        add<CPW, 6>(best, probs, count, nsb, lg_rg);
        add<CPW, 7>(best, probs, count, nsb, lg_rg);
        add<CPW, 8>(best, probs, count, nsb, lg_rg);
    }
    static Plan plan(const GemvProblem *probs, int count, int nsb) {
        Plan best;
        for (int lg_rg = 1; lg_rg <= 3; ++lg_rg) {
            add_v<1>(best, probs, count, nsb, lg_rg);
            add_v<2>(best, probs, count, nsb, lg_rg);
            add_v<3>(best, probs, count, nsb, lg_rg);
        }
        return best;
    }
    template <int CPW, int V>
    static bool go(hipError_t &e, const Plan &pl, const GemvProblem *probs, int count, int nsb,
                   const Prepared &Q, hipStream_t stream) {
        if constexpr (V * CPW <= U) {
            if (pl.cpw == CPW && pl.v == V) {
                e = launch_plan<M, CPW, V, FUSED, RES>(pl, probs, count, nsb, Q, stream);
                return true;
            }
        }
        return false;
    }
    template <int CPW>
    static bool go_v(hipError_t &e, const Plan &pl, const GemvProblem *probs, int count, int nsb,
                     const Prepared &Q, hipStream_t stream) {
        return go<CPW, 1>(e, pl, probs, count, nsb, Q, stream) ||
               go<CPW, 2>(e, pl, probs, count, nsb, Q, stream) ||
               go<CPW, 3>(e, pl, probs, count, nsb, Q, stream) ||
               go<CPW, 4>(e, pl, probs, count, nsb, Q, stream) ||
               go<CPW, 5>(e, pl, probs, count, nsb, Q, stream) ||
               go<CPW, 6>(e, pl, probs, count, nsb, Q, stream) ||
               go<CPW, 7>(e, pl, probs, count, nsb, Q, stream) ||
               go<CPW, 8>(e, pl, probs, count, nsb, Q, stream);
    }
    static hipError_t launch(const Plan &pl, const GemvProblem *probs, int count, int nsb,
                             const Prepared &Q, hipStream_t stream) {
        hipError_t e = hipErrorInvalidValue;
        go_v<1>(e, pl, probs, count, nsb, Q, stream) ||
            go_v<2>(e, pl, probs, count, nsb, Q, stream) ||
            go_v<3>(e, pl, probs, count, nsb, Q, stream);
        return e;
    }
};

// Plans are cached by shape (they depend on the sizes only).
struct PlanKey {
    int64_t N[kMaxGemvBatch];
    int count, nsb, M;
    bool fused;
    bool operator==(const PlanKey &o) const {
        if (count != o.count || nsb != o.nsb || M != o.M || fused != o.fused) return false;
        for (int i = 0; i < count; ++i)
            if (N[i] != o.N[i]) return false;
        return true;
    }
};
struct PlanKeyHash {
    size_t operator()(const PlanKey &k) const {
        size_t h = (size_t)k.count * 1000003u ^ (size_t)k.nsb * 7919u ^ (size_t)k.M * 31u ^
                   (k.fused ? 0x9e3779b9u : 0u);
        for (int i = 0; i < k.count; ++i) h = h * 1315423911u ^ (size_t)k.N[i];
        return h;
    }
};

template <int M, bool FUSED, bool RES>
hipError_t run_m(const GemvProblem *probs, int count, int nsb, const Prepared &Q,
                 hipStream_t stream) {
    static std::mutex mu;
    static std::unordered_map<PlanKey, Plan, PlanKeyHash> cache;
    PlanKey key = {};
    key.count = count;
    key.nsb = nsb;
    key.M = M;
    key.fused = FUSED;
    for (int i = 0; i < count; ++i) key.N[i] = probs[i].N;
    Plan pl;
    {
        std::lock_guard<std::mutex> lock(mu);
        auto it = cache.find(key);
        if (it != cache.end()) {
            pl = it->second;
        } else {
            pl = Table<M, FUSED, RES>::plan(probs, count, nsb);
            if (cache.size() > 4096) cache.clear();
            cache.emplace(key, pl);
        }
    }
    if (!pl.ok) return hipErrorInvalidValue;
    return Table<M, FUSED, RES>::launch(pl, probs, count, nsb, Q, stream);
}

// RES: Q.residual is set (a single product); its kernels are instantiated
// only in the translation unit of the residual entry point.
template <bool FUSED, bool RES = false>
hipError_t run(const GemvProblem *probs, int count, int64_t K, int64_t M, const Prepared &Q,
               hipStream_t stream) {
    const int nsb = (int)(K / kQK);
    switch (M) {
    case 1: return run_m<1, FUSED, RES>(probs, count, nsb, Q, stream);
    case 2: return run_m<2, FUSED, RES>(probs, count, nsb, Q, stream);
    case 3: return run_m<3, FUSED, RES>(probs, count, nsb, Q, stream);
    case 4: return run_m<4, FUSED, RES>(probs, count, nsb, Q, stream);
    case 5: return run_m<5, FUSED, RES>(probs, count, nsb, Q, stream);
    case 6: return run_m<6, FUSED, RES>(probs, count, nsb, Q, stream);
    case 7: return run_m<7, FUSED, RES>(probs, count, nsb, Q, stream);
    case 8: return run_m<8, FUSED, RES>(probs, count, nsb, Q, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace stream
}  // namespace q4k
