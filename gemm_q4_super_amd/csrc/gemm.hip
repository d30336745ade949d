// Prefill GEMM: y[M][N] = Q8(x)[M][K] * W^T with W in Q4_K, any M >= 1.
//
// Prefill is compute-bound ("genie-ai-runtime ...", section 3: batched
// layer-major prefill, Path E tensor-core kernel), so the sub-block integer dot
// products run on the matrix cores.  With x^ = a*c (Q8) and
// w = d*sc[j]*q - dmin*mn[j] (Q4_K), one output is
//
//   y[m][n] = sum_{b,j} a[m,b,j] * (d*sc)[n,b,j] * D[m,n,b,j]
//           - sum_{b,j} (a*S)[m,b,j] * (dmin*mn)[n,b,j]
//
// with D = sum_{i<32} q*c the exact integer dot of one 32-element sub-block and
// S the activation block's code sum.
//
//  * D: one v_mfma_i32_32x32x32_i8 per sub-block and 32 x 32 tile: activation
//    codes (A operand, rows m) against nibble-expanded int8 quants (B operand,
//    columns n), both read from LDS.  Bit-exact.
//  * First sum: fp32 epilogue per sub-block, acc += float(D) * (a * d*sc).
//    Activation and weight scales both change every 32 elements of K, so this
//    costs three VALU operations per output and sub-block: the binding unit.
//  * Second sum (the min term): a contraction over K/32 of fp32 factors, on the
//    bf16 matrix cores with each factor split into two bf16 parts (16
//    significant bits), accumulated over all of K and subtracted at the end.
//  * Workgroup tile BM x BN (one wave per 32 x 32 sub-tile), chosen per shape
//    so that the launch has enough workgroups for 256 CUs.  LDS is
//    double-buffered: the global loads of super-block b+1 are in flight while
//    b is computed, then expanded into the other buffer; one barrier per
//    super-block.
//  * Tile order is XCD-aware: workgroups are dealt round-robin to the 8 XCDs,
//    so all M tiles of one weight column-block are placed on one XCD and run
//    together, sharing that XCD's L2 for the weight rows.
#include "q4k_internal.h"

namespace q4k {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int ROW = 256 + 16;         // padded LDS row of 256 int8 (conflict-free 16-B reads)
constexpr int NXCD = 8;

template <int BM, int BN>
struct __attribute__((aligned(16))) Buf {
    int8_t xq[BM][ROW];               // activation codes
    int8_t wq[BN][ROW];               // weight quants 0..15
    float as[8][BM];                  // activation scale a[m][j]
    float ws[8][BN];                  // d * sc[j]
    unsigned short ph[2][BM][8];      // a*S split hi / lo (bf16 bits)
    unsigned short qh[2][BN][8];      // dmin*mn split hi / lo (bf16 bits)
};

__device__ __forceinline__ float half_lo(unsigned v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFF));
}
__device__ __forceinline__ float half_hi(unsigned v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}
// Split fp32 into two bf16 parts by truncation (hi + lo keeps 16 significant bits).
__device__ __forceinline__ void split_bf16(float v, unsigned short &hi, unsigned short &lo) {
    const unsigned b = __float_as_uint(v);
    hi = (unsigned short)(b >> 16);
    lo = (unsigned short)(__float_as_uint(v - __uint_as_float(b & 0xFFFF0000u)) >> 16);
}

template <int BM, int BN>
struct Cfg {
    static constexpr int WAVES = (BM / 32) * (BN / 32);
    static constexpr int T = 64 * WAVES;
    static constexpr int WCH = 8 * BN;            // 16-B quant chunks of weights per super-block
    static constexpr int XCH = 16 * BM;           // 16-B chunks of activation codes
    static constexpr int SE = 8 * BM;             // activation scale entries
    static constexpr int NW = (WCH + T - 1) / T;
    static constexpr int NX = (XCH + T - 1) / T;
    static constexpr int NS = (SE + T - 1) / T;
};

template <int BM, int BN>
struct Regs {
    u32x4 hd;                         // header of weight row tid (tid < BN)
    u32x4 wc[Cfg<BM, BN>::NW];
    i32x4 xc[Cfg<BM, BN>::NX];
    float a[Cfg<BM, BN>::NS];
    int s[Cfg<BM, BN>::NS];
};

template <int BM, int BN>
__global__ __launch_bounds__((64 * (BM / 32) * (BN / 32))) void gemm_i8_kernel(
    const uint8_t *__restrict__ w, int N, int nsb, const int8_t *__restrict__ codes,
    const float *__restrict__ scales, const int32_t *__restrict__ sums, int M,
    float *__restrict__ y) {
    using C = Cfg<BM, BN>;
    __shared__ Buf<BM, BN> buf[2];

    // XCD-aware tile of this workgroup.
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    const int xcd = blockIdx.x % NXCD, pos = blockIdx.x / NXCD;
    const int nt = (pos / tiles_m) * NXCD + xcd, mt = pos % tiles_m;
    if (nt >= tiles_n) return;   // the whole workgroup exits together, before any barrier
    const int m0 = mt * BM, n0 = nt * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    constexpr int WN = BN / 32;
    const int wm = wave / WN, wn = wave % WN;
    const int K = nsb * 256, nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * 144;
    const int lr = lane & 31, lh = lane >> 5;

    // Global loads of one super-block, branch-free from clamped addresses (a
    // load under a branch makes the compiler wait for every outstanding load
    // at the join, which would drain the prefetch pipeline).  Rows past N or M
    // read row N-1 / M-1: they only feed outputs that are never stored.
    auto load = [&](int b, Regs<BM, BN> &r) {
        {
            const int row = min(n0 + min(tid, BN - 1), N - 1);
            r.hd = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                w + (int64_t)row * row_bytes + (int64_t)b * 144));
        }
#pragma unroll
        for (int i = 0; i < C::NW; ++i) {
            const int e = min(tid + i * C::T, C::WCH - 1);
            const int row = min(n0 + (e >> 3), N - 1), ch = e & 7;
            r.wc[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                w + (int64_t)row * row_bytes + (int64_t)b * 144 + 16 + 16 * ch));
        }
#pragma unroll
        for (int i = 0; i < C::NX; ++i) {
            const int e = min(tid + i * C::T, C::XCH - 1);
            const int row = min(m0 + (e >> 4), M - 1), ch = e & 15;
            r.xc[i] = *reinterpret_cast<const i32x4 *>(codes + (int64_t)row * K + 256 * b + 16 * ch);
        }
#pragma unroll
        for (int i = 0; i < C::NS; ++i) {
            const int e = min(tid + i * C::T, C::SE - 1);
            const int row = min(m0 + (e >> 3), M - 1), j = e & 7;
            const int64_t o = (int64_t)row * nblk + 8 * b + j;
            r.a[i] = scales[o];
            r.s[i] = sums[o];
        }
    };
    auto store = [&](const Regs<BM, BN> &r, Buf<BM, BN> &B) {
        if (tid < BN) {
            // header of weight row tid: fp16 d, dmin and the 6-bit scales/mins
            const u32x4 v = r.hd;
            const float d = half_lo(v.x), dmin = half_hi(v.x);
            const unsigned h1 = v.y, h2 = v.z, h3 = v.w;
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
                B.ws[j][tid] = d * (float)sc;
                unsigned short qhi, qlo;
                split_bf16(dmin * (float)mn, qhi, qlo);
                B.qh[0][tid][j] = qhi;
                B.qh[1][tid][j] = qlo;
            }
        }
#pragma unroll
        for (int i = 0; i < C::NW; ++i) {
            const int e = tid + i * C::T;
            if (e >= C::WCH) continue;
            // quant chunk c: low nibbles -> elements 64g+16h+i, high nibbles ->
            // 64g+32+16h+i (g = c/2, h = c%2)
            const int row = e >> 3, c = e & 7, g = c >> 1, h = c & 1;
            const u32x4 v = r.wc[i];
            u32x4 lo, hi;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                lo[k] = v[k] & 0x0F0F0F0Fu;
                hi[k] = (v[k] >> 4) & 0x0F0F0F0Fu;
            }
            *reinterpret_cast<u32x4 *>(&B.wq[row][64 * g + 16 * h]) = lo;
            *reinterpret_cast<u32x4 *>(&B.wq[row][64 * g + 32 + 16 * h]) = hi;
        }
#pragma unroll
        for (int i = 0; i < C::NX; ++i) {
            const int e = tid + i * C::T;
            if (e < C::XCH)
                *reinterpret_cast<i32x4 *>(&B.xq[e >> 4][16 * (e & 15)]) = r.xc[i];
        }
#pragma unroll
        for (int i = 0; i < C::NS; ++i) {
            const int e = tid + i * C::T;
            if (e >= C::SE) continue;
            const int row = e >> 3, j = e & 7;
            B.as[j][row] = r.a[i];
            unsigned short phi, plo;
            split_bf16(r.a[i] * (float)r.s[i], phi, plo);
            B.ph[0][row][j] = phi;
            B.ph[1][row][j] = plo;
        }
    };

    float acc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.0f;
    f32x16 mins;
#pragma unroll
    for (int i = 0; i < 16; ++i) mins[i] = 0.0f;

    const int am = wm * 32 + lr;      // A operand row (activation) within the tile
    const int bn = wn * 32 + lr;      // B operand column (weight row) within the tile

    // One super-block of work on LDS buffer B.
    auto compute = [&](const Buf<BM, BN> &B) {
#pragma unroll 2
        for (int j = 0; j < 8; ++j) {
            const i32x4 aop = *reinterpret_cast<const i32x4 *>(&B.xq[am][32 * j + 16 * lh]);
            const i32x4 bop = *reinterpret_cast<const i32x4 *>(&B.wq[bn][32 * j + 16 * lh]);
            const i32x16 D = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                aop, bop, (i32x16){0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0}, 0, 0, 0);
            const float wsj = B.ws[j][bn];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const f32x4 a4 =
                    *reinterpret_cast<const f32x4 *>(&B.as[j][wm * 32 + 8 * rr + 4 * lh]);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[4 * rr + t] = fmaf((float)D[4 * rr + t], a4[t] * wsj, acc[4 * rr + t]);
            }
        }
        const bf16x8 pa_h = *reinterpret_cast<const bf16x8 *>(&B.ph[0][am][0]);
        const bf16x8 pa_l = *reinterpret_cast<const bf16x8 *>(&B.ph[1][am][0]);
        const bf16x8 qb = *reinterpret_cast<const bf16x8 *>(&B.qh[lh][bn][0]);
        mins = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_h, qb, mins, 0, 0, 0);
        mins = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa_l, qb, mins, 0, 0, 0);
    };

    // Software pipeline, prefetch distance 2: while super-block b is computed
    // from LDS, the registers hold b+1 (loaded one iteration earlier) and the
    // loads of b+2 are in flight into the other register set.
    Regs<BM, BN> ra, rb;
    load(0, ra);
    store(ra, buf[0]);
    if (nsb > 1) load(1, ra);
    __syncthreads();
    for (int b = 0; b < nsb; b += 2) {
        // even step: compute b from buf[0]; ra holds b+1
        if (b + 2 < nsb) load(b + 2, rb);
        compute(buf[0]);
        if (b + 1 < nsb) store(ra, buf[1]);
        __syncthreads();
        if (b + 1 >= nsb) break;
        // odd step: compute b+1 from buf[1]; rb holds b+2
        if (b + 3 < nsb) load(b + 3, ra);
        compute(buf[1]);
        if (b + 2 < nsb) store(rb, buf[0]);
        __syncthreads();
    }

    const int n = n0 + bn;
    if (n < N) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = m0 + wm * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
            if (m < M) y[(int64_t)m * N + n] = acc[i] - mins[i];
        }
    }
}

template <int BM, int BN>
hipError_t launch_tile(const uint8_t *w, int64_t N, int nsb, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       hipStream_t stream) {
    const int64_t tiles_m = (M + BM - 1) / BM;
    const int64_t tiles_n = (N + BN - 1) / BN;
    const int64_t groups = (tiles_n + NXCD - 1) / NXCD;
    const int64_t grid = groups * NXCD * tiles_m;
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN>), dim3((unsigned)grid), dim3(Cfg<BM, BN>::T), 0,
                       stream, w, (int)N, nsb, codes, scales, sums, (int)M, y);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       hipStream_t stream) {
    const int nsb = (int)(K / kQK);
    // Largest tile that still gives the launch at least half a workgroup per CU.
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (tiles(128, 64) >= 128)
        return launch_tile<128, 64>(w, N, nsb, codes, scales, sums, M, y, stream);
    if (tiles(64, 32) >= 128)
        return launch_tile<64, 32>(w, N, nsb, codes, scales, sums, M, y, stream);
    return launch_tile<32, 32>(w, N, nsb, codes, scales, sums, M, y, stream);
}

}  // namespace q4k
