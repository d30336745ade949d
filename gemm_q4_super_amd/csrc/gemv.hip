// Plain GEMV on prepared Q8 rows (q4k_gemv): y[M][N] = Q8(x)[M][K] * W^T, W in
// Q4_K, M = 1..8.  Where the Q8 rows fit in LDS (M*K <= 32768) the call runs
// the streaming GEMV of stream_gemv.h (the same kernel as the fused
// q4k_quantize_gemv, so the two are bit-identical); wider rows run the kernel
// below, which reads the activation straight from memory.
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
//  * The fused quantize + GEMV (q4k_quantize_gemv, ..._batch) lives in
//    qgemv.hip; this kernel takes prepared Q8 rows (q4k_quantize_act).
#include "stream_gemv.h"

namespace q4k {
namespace {

constexpr int kMaxWaves = 16;

// Kernel arguments: one matrix and its prepared Q8 rows.
struct GemvArgs {
    const uint8_t *w;
    float *y;
    int N;
    const int8_t *codes;
    const float *scales;
    const int32_t *sums;
};

template <int M, int T, int CPW>
__global__ __launch_bounds__(1024) void gemv_kernel(const GemvArgs B, int nsb) {
    __shared__ float red[kMaxWaves][8 * T][M];

    const uint8_t *__restrict__ w = B.w;
    float *__restrict__ y = B.y;
    const int N = B.N;
    const int8_t *__restrict__ codes = B.codes;
    const float *__restrict__ scales = B.scales;
    const int32_t *__restrict__ sums = B.sums;
    asm volatile("" ::"s"(w), "s"(codes), "s"(scales), "s"(sums), "s"(y), "s"(N), "s"(nsb));

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // the launch's wave count, from the kernel arguments (as the host sizes it)
    const int nwaves = (nsb + CPW - 1) / CPW < kMaxWaves ? (nsb + CPW - 1) / CPW : kMaxWaves;
    const int grp = lane >> 3;     // row within a tile of 8
    const LaneMap L(lane & 7);     // chunk index == sub-block owned after the swap
    const int K = nsb * 256;
    const int nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * 144;
    const int row0 = (int)blockIdx.x * (8 * T);

    float acc[T][M];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[t][m] = 0.0f;

    // Columns [b0, b0 + CPW) of this wave; a wave with more than CPW columns
    // (K beyond 16 * CPW super-blocks) takes them in groups of CPW.
    // Activation loads go out before the weight loads where they fit the
    // registers: the load counter retires in order, so data wanted first must
    // be requested first (column 0's dots then overlap the weight stream).
    constexpr bool kActFirst = M * CPW * T <= 6;
    for (int b0 = wave * CPW; b0 < nsb; b0 += nwaves * CPW) {
        i32x4 pA[kActFirst ? CPW : 1][M], pB[kActFirst ? CPW : 1][M];
        float pa[kActFirst ? CPW : 1][M];
        int ps[kActFirst ? CPW : 1][M];   // converted at use, after the loads
        if constexpr (kActFirst) {
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
                hd[c][t] = load_weights16(sb);
                qw[c][t] = load_weights16(sb + 16 + 16 * L.l);
            }
        // Keep every load of the group ahead of the arithmetic below.
        __builtin_amdgcn_sched_barrier(0);
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
                if constexpr (kActFirst) {
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
        if (row < N) y[(int64_t)m * N + row] = v;
    }
}

template <int M, int T, int CPW>
hipError_t launch_mtc(const GemvArgs &B, int nsb, hipStream_t stream) {
    const int nwaves = (nsb + CPW - 1) / CPW < kMaxWaves ? (nsb + CPW - 1) / CPW : kMaxWaves;
    const int tiles = (B.N + 8 * T - 1) / (8 * T);
    hipLaunchKernelGGL((gemv_kernel<M, T, CPW>), dim3(tiles), dim3(64 * nwaves), 0, stream, B,
                       nsb);
    return hipGetLastError();
}

template <int M>
hipError_t launch_m(const GemvArgs &B, int nsb, hipStream_t stream) {
    // Columns per wave: as few as the 16-wave workgroup allows; two row tiles
    // per workgroup once the launch has enough rows to fill the chip.
    if constexpr (M <= 2) {
        if (B.N >= 4096) {
            if (nsb <= 16) return launch_mtc<M, 2, 1>(B, nsb, stream);
            if (nsb <= 32) return launch_mtc<M, 2, 2>(B, nsb, stream);
            return launch_mtc<M, 2, 3>(B, nsb, stream);
        }
    }
    if (nsb <= 16) return launch_mtc<M, 1, 1>(B, nsb, stream);
    if (nsb <= 32) return launch_mtc<M, 1, 2>(B, nsb, stream);
    return launch_mtc<M, 1, 3>(B, nsb, stream);
}

}  // namespace

hipError_t launch_gemv(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       hipStream_t stream) {
    if (gemv_mfma_preferred(N, K, M, scales, sums))
        return launch_gemv_mfma(w, N, K, codes, scales, sums, M, y, stream);
    if (stream_fits(M, K)) {
        const GemvProblem p = {w, nullptr, y, N};
        const stream::Prepared Q = {codes, scales, sums};
        return stream::run<false>(&p, 1, K, M, Q, stream);
    }
    const GemvArgs B = {w, y, (int)N, codes, scales, sums};
    const int nsb = (int)(K / kQK);
    switch (M) {
    case 1: return launch_m<1>(B, nsb, stream);
    case 2: return launch_m<2>(B, nsb, stream);
    case 3: return launch_m<3>(B, nsb, stream);
    case 4: return launch_m<4>(B, nsb, stream);
    case 5: return launch_m<5>(B, nsb, stream);
    case 6: return launch_m<6>(B, nsb, stream);
    case 7: return launch_m<7>(B, nsb, stream);
    case 8: return launch_m<8>(B, nsb, stream);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_batch_prepared(const GemvProblem *probs, int count, int64_t K,
                                      const int8_t *codes, const float *scales,
                                      const int32_t *sums, int64_t M, hipStream_t stream) {
    const stream::Prepared Q = {codes, scales, sums};
    return stream::run<false>(probs, count, K, M, Q, stream);
}

}  // namespace q4k
