// Decode / small-batch GEMV: y[M][N] = Q8(x)[M][K] * W^T, W in Q4_K, M = 1..8.
//
// Batch-1 decode streams every weight byte once and is bound by memory
// bandwidth ("genie-ai-runtime ...", section 2, the decode ceiling), so this
// kernel is built around the HBM stream and uses no matrix cores:
//
//  * Lane <-> 16-byte quant chunk.  A super-block is 144 B = a 16-B header
//    plus eight 16-B quant chunks; 8 lanes (a "group") take one super-block,
//    lane l loading chunk l with one 16-B load and the header with another.
//    Chunk l holds, for g = l/2 and h = l%2, elements 64g+16h+i (low nibbles,
//    sub-block 2g) and 64g+32+16h+i (high nibbles, sub-block 2g+1), i < 16.
//    (The pages' Path C reads four packed quant bytes as one 32-bit load; on
//    gfx950 a lane moves 16 B per load.)
//  * Sub-block integer dots with v_dot4 (sdot4): 8 per lane per super-block and
//    activation row.  The two partner lanes of a chunk pair exchange one half
//    with a DPP quad swap, after which lane l holds the exact int32 dot of
//    sub-block j = l.  Lane l then applies the fp32 epilogue of sub-block l:
//    acc += a_j * (d*sc_j*D_j - dmin*mn_j*S_j).
//  * Workgroup = W waves splitting the K/256 super-block columns of the same
//    8*T rows; group g of every wave owns rows 8t+g.  The activation chunk of a
//    column is loaded once per wave and reused over the T row tiles and all 8
//    groups.  Per-lane sums reduce over the 8 lanes by DPP, then over the W
//    waves through LDS in a fixed order (deterministic, no atomics).
#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

constexpr int kMaxWaves = 16;

template <int M, int T>
__global__ __launch_bounds__(1024) void gemv_kernel(const uint8_t *__restrict__ w, int N,
                                                    int nsb, int cpw,
                                                    const int8_t *__restrict__ codes,
                                                    const float *__restrict__ scales,
                                                    const int32_t *__restrict__ sums,
                                                    float *__restrict__ y) {
    __shared__ float red[kMaxWaves][8 * T][M];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nwaves = blockDim.x >> 6;
    const int grp = lane >> 3;     // row within a tile of 8
    const LaneMap L(lane & 7);     // chunk index == sub-block owned after the swap
    const int K = nsb * 256;
    const int nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * 144;
    const int row0 = blockIdx.x * (8 * T);

    float acc[T][M];
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
        for (int m = 0; m < M; ++m) acc[t][m] = 0.0f;

    const int b_begin = wave * cpw;
    const int b_end = min(nsb, b_begin + cpw);
    for (int b = b_begin; b < b_end; ++b) {
        // Weights of this column for all T row tiles: issue the loads first.
        u32x4 hd[T], qw[T];
#pragma unroll
        for (int t = 0; t < T; ++t) {
            const int row = row0 + 8 * t + grp;
            if (row < N) {
                const uint8_t *sb = w + (int64_t)row * row_bytes + (int64_t)b * 144;
                hd[t] = load_stream16(sb);
                qw[t] = load_stream16(sb + 16 + 16 * L.l);
            } else {
                hd[t] = (u32x4){0u, 0u, 0u, 0u};
                qw[t] = (u32x4){0u, 0u, 0u, 0u};
            }
        }
        // Activation chunk of this column, reused over the row tiles.
        i32x4 cA[M], cB[M];
        float a[M];
        float s[M];
#pragma unroll
        for (int m = 0; m < M; ++m) {
            const int8_t *cm = codes + (int64_t)m * K + 256 * b;
            cA[m] = *reinterpret_cast<const i32x4 *>(cm + L.offA);
            cB[m] = *reinterpret_cast<const i32x4 *>(cm + L.offB);
            a[m] = scales[(int64_t)m * nblk + 8 * b + L.l];
            s[m] = (float)sums[(int64_t)m * nblk + 8 * b + L.l];
        }
#pragma unroll
        for (int t = 0; t < T; ++t) {
            float ds, dm;
            decode_scale(L, hd[t], ds, dm);
            int qlo[4], qhi[4];
            unpack_nibbles(qw[t], qlo, qhi);
#pragma unroll
            for (int m = 0; m < M; ++m) {
                const int D = subblock_dot(L, qlo, qhi, cA[m], cB[m]);
                acc[t][m] = fmaf(a[m], ds * (float)D - dm * s[m], acc[t][m]);
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
    for (int i = threadIdx.x; i < 8 * T * M; i += blockDim.x) {
        const int r = i / M, m = i % M;
        float v = 0.0f;
        for (int wv = 0; wv < nwaves; ++wv) v += red[wv][r][m];
        const int row = row0 + r;
        if (row < N) y[(int64_t)m * N + row] = v;
    }
}

template <int M, int T>
hipError_t launch_mt(const uint8_t *w, int N, int nsb, const int8_t *codes,
                     const float *scales, const int32_t *sums, float *y, hipStream_t stream) {
    int cpw = (nsb + kMaxWaves - 1) / kMaxWaves;
    const int nwaves = (nsb + cpw - 1) / cpw;
    const int rows_per_wg = 8 * T;
    const int grid = (N + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((gemv_kernel<M, T>), dim3(grid), dim3(64 * nwaves), 0, stream, w, N,
                       nsb, cpw, codes, scales, sums, y);
    return hipGetLastError();
}

template <int M>
hipError_t launch_m(const uint8_t *w, int N, int nsb, const int8_t *codes,
                    const float *scales, const int32_t *sums, float *y, hipStream_t stream) {
    // Two row tiles per workgroup once there are enough rows to fill the chip.
    if (N >= 4096 && M <= 4)
        return launch_mt<M, 2>(w, N, nsb, codes, scales, sums, y, stream);
    return launch_mt<M, 1>(w, N, nsb, codes, scales, sums, y, stream);
}

}  // namespace

hipError_t launch_gemv(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       hipStream_t stream) {
    const int nsb = (int)(K / kQK);
    const int n = (int)N;
    switch (M) {
    case 1: return launch_m<1>(w, n, nsb, codes, scales, sums, y, stream);
    case 2: return launch_m<2>(w, n, nsb, codes, scales, sums, y, stream);
    case 3: return launch_m<3>(w, n, nsb, codes, scales, sums, y, stream);
    case 4: return launch_m<4>(w, n, nsb, codes, scales, sums, y, stream);
    case 5: return launch_m<5>(w, n, nsb, codes, scales, sums, y, stream);
    case 6: return launch_m<6>(w, n, nsb, codes, scales, sums, y, stream);
    case 7: return launch_m<7>(w, n, nsb, codes, scales, sums, y, stream);
    case 8: return launch_m<8>(w, n, nsb, codes, scales, sums, y, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace q4k
