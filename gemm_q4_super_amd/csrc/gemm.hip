// Prefill GEMM: y[M][N] = Q8(x)[M][K] * W^T with W in Q4_K, any M >= 1.
//
// Prefill is compute-bound ("genie-ai-runtime ...", section 3: batched
// layer-major prefill, Path E tensor-core kernel), so the sub-block integer dot
// products run on the matrix cores:
//
//  * Workgroup tile BM x BN = 64 x 64 outputs, 4 waves of 32 x 32.
//  * Per super-block (256 of K): the 64 weight rows are read once (144 B each)
//    and nibble-expanded into LDS as int8 quants (q in 0..15), with the fp32
//    factors d*sc[j] and dmin*mn[j] of every row and sub-block; the activation
//    scales a[m][j] and a[m][j]*S[m][j] of the 64 activation rows are staged
//    beside them.
//  * Per 32-element sub-block j: one v_mfma_i32_32x32x32_i8 per wave gives the
//    exact int32 dots D[m][n] = sum q*c of its 32 x 32 tile; the fp32 epilogue
//    adds a[m][j]*(d*sc[j])*D - (a*S)[m][j]*(dmin*mn[j]).
//
// The weight quants and activation codes are exact small integers, so D is
// bit-exact; the fp32 epilogue differs from the plain sum only in rounding.
#include "q4k_internal.h"

namespace q4k {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 64, BN = 64;
constexpr int BQ_STRIDE = 256 + 16;   // padded LDS row (bank-conflict-free 16-B reads)

__device__ __forceinline__ float half_lo(unsigned v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFF));
}
__device__ __forceinline__ float half_hi(unsigned v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}

__global__ __launch_bounds__(256) void gemm_i8_kernel(const uint8_t *__restrict__ w, int N,
                                                      int nsb,
                                                      const int8_t *__restrict__ codes,
                                                      const float *__restrict__ scales,
                                                      const int32_t *__restrict__ sums, int M,
                                                      float *__restrict__ y) {
    __shared__ __attribute__((aligned(16))) int8_t Bq[BN][BQ_STRIDE];
    __shared__ float Ws[BN][8];      // d * sc[j]
    __shared__ float Wm[BN][8];      // dmin * mn[j]
    __shared__ __attribute__((aligned(16))) float As[8][BM];   // a[m][j]
    __shared__ __attribute__((aligned(16))) float Ap[8][BM];   // a[m][j] * S[m][j]

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int tiles_n = (N + BN - 1) / BN;
    const int m0 = (blockIdx.x / tiles_n) * BM, n0 = (blockIdx.x % tiles_n) * BN;
    const int K = nsb * 256, nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * 144;

    // staging roles
    const int sr = tid >> 2, sq = tid & 3;        // weight row, chunk pair
    const int an = n0 + sr;                       // weight row index
    // MFMA operand roles
    const int lr = lane & 31, lh = lane >> 5;
    const int am = m0 + wm * 32 + lr;             // activation row of the A operand

    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;

    for (int b = 0; b < nsb; ++b) {
        // Global loads for this super-block.
        u32x4 q0 = {0u, 0u, 0u, 0u}, q1 = {0u, 0u, 0u, 0u}, hd = {0u, 0u, 0u, 0u};
        if (an < N) {
            const uint8_t *sb = w + (int64_t)an * row_bytes + (int64_t)b * 144;
            q0 = *reinterpret_cast<const u32x4 *>(sb + 16 + 32 * sq);
            q1 = *reinterpret_cast<const u32x4 *>(sb + 32 + 32 * sq);
            if (sq == 0) hd = *reinterpret_cast<const u32x4 *>(sb);
        }
        i32x4 aop[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (am < M)
                aop[j] = *reinterpret_cast<const i32x4 *>(codes + (int64_t)am * K + 256 * b +
                                                          32 * j + 16 * lh);
            else
                aop[j] = (i32x4){0, 0, 0, 0};
        }
        float sa0 = 0.0f, sp0 = 0.0f, sa1 = 0.0f, sp1 = 0.0f;
        {
            // 512 (m, j) activation-scale entries, two per thread.
            const int e0 = tid, e1 = tid + 256;
            const int m_a = e0 >> 3, j_a = e0 & 7, m_b = e1 >> 3, j_b = e1 & 7;
            if (m0 + m_a < M) {
                const int64_t o = (int64_t)(m0 + m_a) * nblk + 8 * b + j_a;
                sa0 = scales[o];
                sp0 = sa0 * (float)sums[o];
            }
            if (m0 + m_b < M) {
                const int64_t o = (int64_t)(m0 + m_b) * nblk + 8 * b + j_b;
                sa1 = scales[o];
                sp1 = sa1 * (float)sums[o];
            }
        }

        __syncthreads();   // the previous super-block's LDS reads are done
        // Nibble-expand chunks 2*sq and 2*sq+1 of row sr into int8 quants.
        {
            const u32x4 qq[2] = {q0, q1};
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                const int c = 2 * sq + c2, g = c >> 1, h = c & 1;
                u32x4 lo, hi;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    lo[k] = qq[c2][k] & 0x0F0F0F0Fu;
                    hi[k] = (qq[c2][k] >> 4) & 0x0F0F0F0Fu;
                }
                *reinterpret_cast<u32x4 *>(&Bq[sr][64 * g + 16 * h]) = lo;
                *reinterpret_cast<u32x4 *>(&Bq[sr][64 * g + 32 + 16 * h]) = hi;
            }
            if (sq == 0) {
                const float d = half_lo(hd.x), dmin = half_hi(hd.x);
                const unsigned h1 = hd.y, h2 = hd.z, h3 = hd.w;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    unsigned sc, mn;
                    if (j < 4) {
                        sc = (h1 >> (8 * j)) & 63u;
                        mn = (h2 >> (8 * j)) & 63u;
                    } else {
                        const int s = 8 * (j - 4);
                        sc = ((h3 >> s) & 15u) | (((h1 >> (s + 6)) & 3u) << 4);
                        mn = ((h3 >> (s + 4)) & 15u) | (((h2 >> (s + 6)) & 3u) << 4);
                    }
                    Ws[sr][j] = d * (float)sc;
                    Wm[sr][j] = dmin * (float)mn;
                }
            }
            As[tid & 7][tid >> 3] = sa0;
            Ap[tid & 7][tid >> 3] = sp0;
            As[(tid + 256) & 7][(tid + 256) >> 3] = sa1;
            Ap[(tid + 256) & 7][(tid + 256) >> 3] = sp1;
        }
        __syncthreads();

        const int bn = wn * 32 + lr;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const i32x4 bop = *reinterpret_cast<const i32x4 *>(&Bq[bn][32 * j + 16 * lh]);
            const i32x16 zero = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
            const i32x16 D = __builtin_amdgcn_mfma_i32_32x32x32_i8(aop[j], bop, zero, 0, 0, 0);
            const float ws = Ws[bn][j], wmn = Wm[bn][j];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int mb = wm * 32 + 8 * r + 4 * lh;
                const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&As[j][mb]);
                const f32x4 p4 = *reinterpret_cast<const f32x4 *>(&Ap[j][mb]);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int i = 4 * r + t;
                    acc[i] = fmaf((float)D[i], a4[t] * ws, acc[i]);
                    acc[i] = fmaf(-p4[t], wmn, acc[i]);
                }
            }
        }
    }

    const int n = n0 + wn * 32 + lr;
    if (n < N) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + wm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
            if (m < M) y[(int64_t)m * N + n] = acc[i];
        }
    }
}

}  // namespace

hipError_t launch_gemm(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       hipStream_t stream) {
    const int nsb = (int)(K / kQK);
    const int64_t tiles = ((N + BN - 1) / BN) * ((M + BM - 1) / BM);
    dim3 grid((unsigned)tiles);
    hipLaunchKernelGGL(gemm_i8_kernel, grid, dim3(256), 0, stream, w, (int)N, nsb, codes, scales,
                       sums, (int)M, y);
    return hipGetLastError();
}

}  // namespace q4k
