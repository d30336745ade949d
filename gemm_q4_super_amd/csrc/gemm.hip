// Prefill GEMM: y[M][N] = Q8(x)[M][K] * W^T with W in Q4_K, any M >= 1.
//
// Prefill is compute-bound ("genie-ai-runtime ...", section 3: batched
// layer-major prefill, Path E tensor-core kernel), so the contraction runs on
// the matrix cores.  With x^ = a*c (Q8: one fp32 scale a per 32 codes c) and
// w = d*sc[j]*q - dmin*mn[j] (Q4_K), one output is
//
//   y[m][n] = sum_b d[n,b] * sum_{k in b} (sc*q)[n,k] * x^[m,k]
//           - sum_{b,j} (dmin*mn)[n,b,j] * (a*S)[m,b,j]
//
// with S the code sum of one activation block.
//
// Both per-32-element scales sit inside the matrix-core operands, so the
// only vector-ALU work per output is one fma per super-block:
//  * weight operand (B, columns n): the integer sc*q <= 945, exact in fp16, made
//    from the nibbles with one byte permute and one packed fp16 fma per pair
//    ((1024 + q)*sc - 1024*sc, fused, so exact);
//  * activation operand (A, rows m): x^ scaled by a power of two 2^-e per
//    activation row and super-block (e from the largest block scale, which
//    keeps every value in fp16 range), split into two fp16 parts hi + lo
//    with 22 significant bits: hi = fp16(c*ah) and lo = fp16((c*ah - hi) +
//    c*al) where a*2^-e = ah + al; c*ah - hi is exact in fp16 (the error of
//    an fp16 product), so hi + lo = a*2^-e*c to about 2^-21;
//  * sc*q*hi and sc*q*lo products are exact in fp32; each super-block's sum
//    accumulates over 16 v_mfma_f32_32x32x16_f16 per 32x32 tile, then
//    acc += (d * 2^e) * tmp;
//  * min term: bf16 matrix cores with both fp32 factors split into two bf16
//    parts (16 significant bits), accumulated straight into acc.
// Activation scales make an int8 contraction cost three vector operations
// per output and 32 elements (convert, scale product, fma); on gfx950 those
// do not overlap with the matrix cores, which is why this path spends
// twice the fp16 matrix work instead.
//
// Staging: a quarter super-block (64 elements of K: two sub-blocks, which
// share one 32-byte group of quant bytes) per step, double-buffered in LDS.
// The waves are specialised: on each SIMD one wave only reads operands from
// LDS and runs the matrix-core ops, and one only loads raw blocks from
// global memory and converts them into the other LDS buffer (raw loads two
// steps ahead, two register sets).  A wave that mixes both stalls its vector
// ops behind its own matrix ops, while two waves on one SIMD overlap them.
// One barrier per step.  Workgroup tile (64*WVN) x (32*TM*WVM), one
// matrix-core wave per 64 x 32*TM outputs.  Tile order is XCD-aware: all M
// tiles of one weight column-block run on one XCD, sharing its L2.
#include <algorithm>
#include <type_traits>

#include "q4k_internal.h"

namespace q4k {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NXCD = 8;
constexpr int TN = 2;        // 32-row weight tiles per wave
constexpr int ASTR = 72;     // fp16 per weight row and step: [kh 2][sub 2][lh 2][8] + 8 pad
constexpr int BSTR = 136;    // fp16 per activation row and step: [lh 2][sub 2][kh 2][hi/lo 2][8] + 8 pad

template <int WN, int WM>
struct __attribute__((aligned(16))) Lds {
    _Float16 aw[2][WN][ASTR];        // sc*q of a step's two sub-blocks
    _Float16 bx[2][WM][BSTR];        // x^ * 2^-e as hi, lo
    float dn[2][WN];                 // d of the super-block (by super-block parity)
    float es[2][WM];                 // 2^e of the activation row's super-block
    unsigned short qh[2][2][WN][8];  // -(dmin*mn) split hi / lo (bf16 bits)
    unsigned short ph[2][2][WM][8];  // a*S split hi / lo (bf16 bits)
};

template <int V>
using IC = std::integral_constant<int, V>;

// Products sharing one activation, launched together: product i has N[i]
// weight rows and owns the virtual column-blocks tile0[i] .. tile0[i+1]-1.
struct GemmSet {
    const uint8_t *w[kMaxGemmBatch];
    float *y[kMaxGemmBatch];
    int N[kMaxGemmBatch];
    int tile0[kMaxGemmBatch + 1];
    int count;
};

template <int WVN, int WVM, int TM>
struct Cfg {
    static constexpr int WN = 32 * TN * WVN;
    static constexpr int WM = 32 * TM * WVM;
    static constexpr int NC = WVN * WVM;           // matrix-core waves (as many converting waves)
    static constexpr int P = 64 * NC;              // converting lanes
    static constexpr int T = 2 * P;
    static constexpr int CA = 2 * WN;              // 16-byte quant chunks per step
    static constexpr int CB = 2 * WM;              // 32-code activation blocks per step
    static constexpr int NA = (CA + P - 1) / P;
    static constexpr int NB = (CB + P - 1) / P;
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
// Two fp16 of the integers 1024 + (byte 0, byte 1) or (byte 2, byte 3) of v
// (0x64 is the high byte of fp16 1024, whose unit in the last place is 1).
__device__ __forceinline__ half2 bias_pair_lo(unsigned v) {
    return __builtin_bit_cast(half2, __builtin_amdgcn_perm(0x64646464u, v, 0x04010400u));
}
__device__ __forceinline__ half2 bias_pair_hi(unsigned v) {
    return __builtin_bit_cast(half2, __builtin_amdgcn_perm(0x64646464u, v, 0x04030402u));
}
__device__ __forceinline__ half8 cat4(half2 a, half2 b, half2 c, half2 d) {
    return (half8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}
// 6-bit scale (or min, with hi = true) of sub-block j from the header dwords.
template <int J>
__device__ __forceinline__ unsigned scale6(const u32x4 &h, bool min) {
    const unsigned lo = min ? h.z : h.y;
    if (J < 4) return (lo >> (8 * J)) & 63u;
    const int sh = 8 * (J - 4);
    return ((h.w >> (sh + (min ? 4 : 0))) & 15u) | (((lo >> (sh + 6)) & 3u) << 4);
}

template <int WVN, int WVM, int TM>
__global__ __launch_bounds__(128 * WVN * WVM, 1) void gemm_f16_kernel(
    const GemmSet set, int nsb, const int8_t *__restrict__ codes,
    const float *__restrict__ scales, const int32_t *__restrict__ sums, int M, int splits) {
    using C = Cfg<WVN, WVM, TM>;
    constexpr int WN = C::WN, WM = C::WM, P = C::P;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    Lds<WN, WM> &L = *reinterpret_cast<Lds<WN, WM> *>(lds_raw);

    // XCD-aware tile and K range of this workgroup: the M tiles and K parts
    // of one (virtual) weight column-block run on one XCD.
    const int tiles_m = (M + WM - 1) / WM;
    const int xcd = blockIdx.x % NXCD, pos = blockIdx.x / NXCD;
    const int per = tiles_m * splits;
    const int vt = (pos / per) * NXCD + xcd, mt = (pos % per) / splits, sp = pos % splits;
    if (vt >= set.tile0[set.count]) return;   // the whole workgroup exits, before any barrier
    int pi = 0;
#pragma unroll
    for (int k = 1; k < kMaxGemmBatch; ++k) pi += (k < set.count && vt >= set.tile0[k]);
    const uint8_t *__restrict__ w = set.w[pi];
    float *__restrict__ y = set.y[pi];
    const int N = set.N[pi];
    const int n0 = (vt - set.tile0[pi]) * WN, m0 = mt * WM;
    const int sb0 = (int)((int64_t)nsb * sp / splits);
    const int nl = (int)((int64_t)nsb * (sp + 1) / splits) - sb0;   // >= 1 (splits <= nsb)
    const int K = nsb * 256, nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * 144;
    const int tid = threadIdx.x;

    if (tid >= P) {
        // ---------------- converting waves ----------------
        const int p = tid - P;
        // Raw loads.  Rows past N or M read row N-1 / M-1 and steps past the
        // end of the K range read its last super-block (branch-free loads):
        // they only feed outputs or buffers that are never used.
        struct Step {                 // one step: quant bytes, activation codes
            u32x4 q[C::NA];
            i32x4 c0[C::NB], c1[C::NB];
        };
        struct Block {                // one super-block: headers, block scales and sums
            u32x4 h[C::NA];
            float a[C::NB][8];
            int s[C::NB][8];
        };
        Step S0, S1;
        Block cur, nxt;

        auto load = [&](auto setc, auto gc, int b) {
            constexpr int g = decltype(gc)::value;
            Step &R = decltype(setc)::value ? S1 : S0;
            b = sb0 + min(b, nl - 1);
#pragma unroll
            for (int i = 0; i < C::NA; ++i) {
                const int e = min(p + i * P, C::CA - 1);
                const int row = min(n0 + (e >> 1), N - 1);
                const uint8_t *src = w + (int64_t)row * row_bytes + (int64_t)b * 144;
                R.q[i] = *reinterpret_cast<const u32x4 *>(src + 16 + 32 * g + 16 * (e & 1));
                if (g == 0) nxt.h[i] = *reinterpret_cast<const u32x4 *>(src);
            }
#pragma unroll
            for (int i = 0; i < C::NB; ++i) {
                const int e = min(p + i * P, C::CB - 1);
                const int row = min(m0 + (e >> 1), M - 1);
                const int8_t *src = codes + (int64_t)row * K + 256 * b + 32 * (2 * g + (e & 1));
                R.c0[i] = *reinterpret_cast<const i32x4 *>(src);
                R.c1[i] = *reinterpret_cast<const i32x4 *>(src + 16);
                if (g == 0) {
                    const int64_t o = (int64_t)row * nblk + 8 * b;
                    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(scales + o);
                    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(scales + o + 4);
                    const i32x4 s0 = *reinterpret_cast<const i32x4 *>(sums + o);
                    const i32x4 s1 = *reinterpret_cast<const i32x4 *>(sums + o + 4);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        nxt.a[i][k] = a0[k];
                        nxt.a[i][4 + k] = a1[k];
                        nxt.s[i][k] = s0[k];
                        nxt.s[i][4 + k] = s1[k];
                    }
                }
            }
        };

        // Step g of a super-block (raw step in a register set, super-block data
        // in B) -> LDS buffer F and super-block parity Q.  The weight quants
        // become fp16 sc*q (and, on the first step, d and the min factors are
        // written); the activation codes become fp16 hi, lo.  Lanes that share
        // a row write identical header values.
        auto convert = [&](auto setc, auto gc, auto bufc, const Block &B, int Q) {
            constexpr int g = decltype(gc)::value;
            constexpr int F = decltype(bufc)::value;
            const Step &R = decltype(setc)::value ? S1 : S0;
#pragma unroll
            for (int i = 0; i < C::NA; ++i) {
                const int e = p + i * P;
                if (C::CA % P != 0 && e >= C::CA) continue;   // (no branch when the chunks tile the lanes)
                const int row = e >> 1, c = e & 1;
                const u32x4 h = B.h[i], q = R.q[i];
                // low nibbles: sub-block 2g, high nibbles: sub-block 2g+1; byte t
                // of the chunk is element 16c + t of both
                const float sc0 = (float)scale6<2 * g>(h, false), sc1 = (float)scale6<2 * g + 1>(h, false);
                const half2 sv0 = {(_Float16)sc0, (_Float16)sc0};
                const half2 bv0 = {(_Float16)(-1024.0f * sc0), (_Float16)(-1024.0f * sc0)};
                const half2 sv1 = {(_Float16)sc1, (_Float16)sc1};
                const half2 bv1 = {(_Float16)(-1024.0f * sc1), (_Float16)(-1024.0f * sc1)};
                u32x4 lo, hi;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    lo[k] = q[k] & 0x0F0F0F0Fu;
                    hi[k] = (q[k] >> 4) & 0x0F0F0F0Fu;
                }
                auto conv = [&](unsigned v0, unsigned v1, half2 sv, half2 bv) {
                    return cat4(__builtin_elementwise_fma(bias_pair_lo(v0), sv, bv),
                                __builtin_elementwise_fma(bias_pair_hi(v0), sv, bv),
                                __builtin_elementwise_fma(bias_pair_lo(v1), sv, bv),
                                __builtin_elementwise_fma(bias_pair_hi(v1), sv, bv));
                };
                // kh = c; the two lanes of a row land 16 banks apart (no conflict)
                _Float16 *dst = &L.aw[F][row][32 * c];
                *reinterpret_cast<half8 *>(dst + 0) = conv(lo.x, lo.y, sv0, bv0);
                *reinterpret_cast<half8 *>(dst + 8) = conv(lo.z, lo.w, sv0, bv0);
                *reinterpret_cast<half8 *>(dst + 16) = conv(hi.x, hi.y, sv1, bv1);
                *reinterpret_cast<half8 *>(dst + 24) = conv(hi.z, hi.w, sv1, bv1);
                if (g == 0) {
                    L.dn[Q][row] = half_lo(h.x);
                    const float dmin = half_hi(h.x);
                    // part c of the bf16 split: c = 0 the truncated high half, c = 1 the rest
                    auto part = [&](unsigned mn) -> unsigned {
                        const float v = -dmin * (float)mn;
                        const unsigned bits = __float_as_uint(v);
                        const float r = v - __uint_as_float(bits & 0xFFFF0000u);
                        return (c ? __float_as_uint(r) : bits) >> 16;
                    };
                    u32x4 pv;
                    pv[0] = part(scale6<0>(h, true)) | (part(scale6<1>(h, true)) << 16);
                    pv[1] = part(scale6<2>(h, true)) | (part(scale6<3>(h, true)) << 16);
                    pv[2] = part(scale6<4>(h, true)) | (part(scale6<5>(h, true)) << 16);
                    pv[3] = part(scale6<6>(h, true)) | (part(scale6<7>(h, true)) << 16);
                    *reinterpret_cast<u32x4 *>(&L.qh[Q][c][row][0]) = pv;
                }
            }
            const half2 m1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
            for (int i = 0; i < C::NB; ++i) {
                const int e = p + i * P;
                if (C::CB % P != 0 && e >= C::CB) continue;
                const int row = e >> 1, jb = e & 1;
                // power-of-two scaling of the row's super-block: largest scale in [1, 2)
                float amax = B.a[i][0];
#pragma unroll
                for (int k = 1; k < 8; ++k) amax = fmaxf(amax, B.a[i][k]);
                const int ex = amax > 0.0f ? __builtin_amdgcn_frexp_expf(amax) - 1 : 0;
                // block 2g + jb's scale and sum, as bit selects (an indexed read
                // would go to scratch)
                const unsigned msk = 0u - (unsigned)jb;
                const float a = __uint_as_float((__float_as_uint(B.a[i][2 * g]) & ~msk) |
                                                (__float_as_uint(B.a[i][2 * g + 1]) & msk));
                const int sj = (B.s[i][2 * g] & (int)~msk) | (B.s[i][2 * g + 1] & (int)msk);
                const float as = __builtin_ldexpf(a, -ex);
                const _Float16 ah = (_Float16)as;
                const _Float16 al = (_Float16)(as - (float)ah);
                const half2 ah2 = {ah, ah}, al2 = {al, al};
                // 8 codes -> hi, lo
                auto conv = [&](unsigned v0, unsigned v1, half8 &hv, half8 &lv) {
                    const unsigned u0 = v0 ^ 0x80808080u, u1 = v1 ^ 0x80808080u;
                    const half2 cc[4] = {bias_pair_lo(u0) + m1152, bias_pair_hi(u0) + m1152,
                                         bias_pair_lo(u1) + m1152, bias_pair_hi(u1) + m1152};
                    half2 hh[4], ll[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        hh[k] = cc[k] * ah2;
                        const half2 r = __builtin_elementwise_fma(cc[k], ah2, -hh[k]);
                        ll[k] = __builtin_elementwise_fma(cc[k], al2, r);
                    }
                    hv = cat4(hh[0], hh[1], hh[2], hh[3]);
                    lv = cat4(ll[0], ll[1], ll[2], ll[3]);
                };
                // sub-block jb; the two lanes of a row land 16 banks apart
                _Float16 *dst = &L.bx[F][row][32 * jb];
                const i32x4 c0 = R.c0[i], c1 = R.c1[i];
                half8 hv, lv;
                conv(c0.x, c0.y, hv, lv);   // elements 0..7: lh 0, kh 0
                *reinterpret_cast<half8 *>(dst + 0) = hv;
                *reinterpret_cast<half8 *>(dst + 8) = lv;
                conv(c0.z, c0.w, hv, lv);   // elements 8..15: lh 1, kh 0
                *reinterpret_cast<half8 *>(dst + 64) = hv;
                *reinterpret_cast<half8 *>(dst + 72) = lv;
                conv(c1.x, c1.y, hv, lv);   // elements 16..23: lh 0, kh 1
                *reinterpret_cast<half8 *>(dst + 16) = hv;
                *reinterpret_cast<half8 *>(dst + 24) = lv;
                conv(c1.z, c1.w, hv, lv);   // elements 24..31: lh 1, kh 1
                *reinterpret_cast<half8 *>(dst + 80) = hv;
                *reinterpret_cast<half8 *>(dst + 88) = lv;
                if (g == 0) L.es[Q][row] = __builtin_ldexpf(1.0f, ex);   // both lanes of the row
                unsigned short phi, plo;
                split_bf16(a * (float)sj, phi, plo);
                L.ph[Q][0][row][2 * g + jb] = phi;
                L.ph[Q][1][row][2 * g + jb] = plo;
            }
        };

        // Per step s: load step s+2 into the register set step s used,
        // convert step s+1 into LDS buffer (s+1) & 1, one barrier.
        load(IC<0>{}, IC<0>{}, 0);
        load(IC<1>{}, IC<1>{}, 0);
        cur = nxt;
        convert(IC<0>{}, IC<0>{}, IC<0>{}, cur, 0);
        __syncthreads();
#pragma unroll 1
        for (int b = 0; b < nl; ++b) {
            const int Q = b & 1;
            load(IC<0>{}, IC<2>{}, b);
            convert(IC<1>{}, IC<1>{}, IC<1>{}, cur, Q);
            __syncthreads();
            load(IC<1>{}, IC<3>{}, b);
            convert(IC<0>{}, IC<2>{}, IC<0>{}, cur, Q);
            __syncthreads();
            load(IC<0>{}, IC<0>{}, b + 1);
            convert(IC<1>{}, IC<3>{}, IC<1>{}, cur, Q);
            __syncthreads();
            load(IC<1>{}, IC<1>{}, b + 1);
            convert(IC<0>{}, IC<0>{}, IC<0>{}, nxt, Q ^ 1);
            __syncthreads();
            cur = nxt;
        }
        return;
    }

    // ---------------- matrix-core waves ----------------
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave / WVM, wm = wave % WVM;
    const int lr = lane & 31, lh = lane >> 5;

    f32x16 acc[TN][TM], tmp[TN][TM];
#pragma unroll
    for (int u = 0; u < TN; ++u)
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                acc[u][t][i] = 0.0f;
                tmp[u][t][i] = 0.0f;
            }

    // Sub-block s of the step in LDS buffer F: 8 matrix-core ops per 32x32 tile.
    auto compute = [&](auto bufc, int s) {
        constexpr int F = decltype(bufc)::value;
        half8 A[TN][2], B[TM][2][2];
#pragma unroll
        for (int u = 0; u < TN; ++u) {
            const _Float16 *src = &L.aw[F][wn * 64 + u * 32 + lr][16 * s + 8 * lh];
            A[u][0] = *reinterpret_cast<const half8 *>(src);
            A[u][1] = *reinterpret_cast<const half8 *>(src + 32);
        }
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const _Float16 *src = &L.bx[F][(wm * TM + t) * 32 + lr][64 * lh + 32 * s];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int hl = 0; hl < 2; ++hl)
                    B[t][kh][hl] = *reinterpret_cast<const half8 *>(src + 16 * kh + 8 * hl);
        }
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int hl = 0; hl < 2; ++hl)
#pragma unroll
                for (int u = 0; u < TN; ++u)
#pragma unroll
                    for (int t = 0; t < TM; ++t)
                        tmp[u][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            B[t][kh][hl], A[u][kh], tmp[u][t], 0, 0, 0);
    };

    // End of a super-block: acc += (d * 2^e) * tmp, and the min term.  A
    // lane's outputs share one weight row n (its d) and span 16 activation
    // rows m (their 2^e).
    auto finish = [&](int Q) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int x0 = (wm * TM + t) * 32;
            float ev[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 e4 = *reinterpret_cast<const f32x4 *>(&L.es[Q][x0 + 8 * q + 4 * lh]);
#pragma unroll
                for (int k = 0; k < 4; ++k) ev[4 * q + k] = e4[k];
            }
            const bf16x8 pa = *reinterpret_cast<const bf16x8 *>(&L.ph[Q][lh][x0 + lr][0]);
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const int r = wn * 64 + u * 32 + lr;
                const float dv = L.dn[Q][r];
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    acc[u][t][i] = fmaf(dv * ev[i], tmp[u][t][i], acc[u][t][i]);
                    tmp[u][t][i] = 0.0f;
                }
                const bf16x8 qh = *reinterpret_cast<const bf16x8 *>(&L.qh[Q][0][r][0]);
                const bf16x8 ql = *reinterpret_cast<const bf16x8 *>(&L.qh[Q][1][r][0]);
                acc[u][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, qh, acc[u][t], 0, 0, 0);
                acc[u][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pa, ql, acc[u][t], 0, 0, 0);
            }
        }
    };

    __syncthreads();
#pragma unroll 1
    for (int b = 0; b < nl; ++b) {
        compute(IC<0>{}, 0);
        compute(IC<0>{}, 1);
        __syncthreads();
        compute(IC<1>{}, 0);
        compute(IC<1>{}, 1);
        __syncthreads();
        compute(IC<0>{}, 0);
        compute(IC<0>{}, 1);
        __syncthreads();
        compute(IC<1>{}, 0);
        compute(IC<1>{}, 1);
        finish(b & 1);
        __syncthreads();
    }

    // Lanes 0..31 hold 32 consecutive n of one activation row: coalesced
    // stores, or (K split over several workgroups) fp32 atomic adds into the
    // zero-filled output.
#pragma unroll
    for (int u = 0; u < TN; ++u) {
        const int n = n0 + wn * 64 + u * 32 + lr;
        if (n >= N) continue;
#pragma unroll
        for (int t = 0; t < TM; ++t)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = m0 + (wm * TM + t) * 32 + 8 * (i >> 2) + 4 * lh + (i & 3);
                if (m >= M) continue;
                float *dst = y + (int64_t)m * N + n;
                if (splits == 1)
                    *dst = acc[u][t][i];
                else
                    unsafeAtomicAdd(dst, acc[u][t][i]);
            }
    }
}

// Zero fill of the outputs before K parts add into them: 16-byte stores
// where an output is 16-byte aligned, else 4-byte stores.
__global__ __launch_bounds__(256) void zero_kernel(const GemmSet set, int64_t M) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    const int64_t i0 = (int64_t)blockIdx.x * 256 + threadIdx.x;
    for (int p = 0; p < set.count; ++p) {
        float *y = set.y[p];
        const int64_t n = M * set.N[p];
        if ((reinterpret_cast<uintptr_t>(y) & 15) == 0) {
            f32x4 *y4 = reinterpret_cast<f32x4 *>(y);
            for (int64_t i = i0; i < n / 4; i += stride) y4[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
            if (i0 < (n & 3)) y[(n & ~(int64_t)3) + i0] = 0.0f;
        } else {
            for (int64_t i = i0; i < n; i += stride) y[i] = 0.0f;
        }
    }
}

template <int WVN, int WVM, int TM>
hipError_t launch_tile(const GemmSet &set, int nsb, const int8_t *codes, const float *scales,
                       const int32_t *sums, int64_t M, int splits, hipStream_t stream) {
    using C = Cfg<WVN, WVM, TM>;
    if (splits > 1) {
        int64_t items = 0;
        for (int p = 0; p < set.count; ++p) items = std::max<int64_t>(items, M * set.N[p] / 4 + 1);
        const int64_t blocks = std::min<int64_t>((items + 255) / 256, 2048);
        hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, set, M);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t tiles_m = (M + C::WM - 1) / C::WM;
    const int64_t groups = (set.tile0[set.count] + NXCD - 1) / NXCD;
    const int64_t grid = groups * NXCD * tiles_m * splits;
    hipLaunchKernelGGL((gemm_f16_kernel<WVN, WVM, TM>), dim3((unsigned)grid), dim3(C::T),
                       sizeof(Lds<C::WN, C::WM>), stream, set, nsb, codes, scales, sums, (int)M,
                       splits);
    return hipGetLastError();
}

// Number of K parts: fill the CUs (one workgroup each) without paying more
// for the zero fill and the atomic adds than the split saves.  Workgroups
// are dealt to the XCDs by weight column-block, so the busiest XCD decides
// the number of rounds.  Costs in microseconds: one quarter super-block step
// of a round ~1.3, the zero fill ~5, the atomic adds ~1.3 bytes per ps.
int choose_splits(int64_t tiles_n, int64_t tiles_m, int nsb, int64_t tile_outputs) {
    const int64_t per_xcd = (cu_count() + NXCD - 1) / NXCD;
    const int64_t cols = (tiles_n + NXCD - 1) / NXCD;   // column-blocks on the busiest XCD
    int best = 1;
    double best_t = 1e30;
    for (int s = 1; s <= 8 && s <= nsb; ++s) {
        const int64_t rounds = (cols * tiles_m * s + per_xcd - 1) / per_xcd;
        const int steps = 4 * ((nsb + s - 1) / s);
        double t = 1.3 * (double)(rounds * steps);
        if (s > 1) t += 5.0 + 4.0 * (double)(tiles_n * tiles_m * s * tile_outputs) / 1.3e6;
        if (t < best_t) {
            best_t = t;
            best = s;
        }
    }
    return best;
}

}  // namespace

hipError_t launch_gemm_batch(const GemmProblem *probs, int count, int64_t K,
                             const int8_t *codes, const float *scales, const int32_t *sums,
                             int64_t M, hipStream_t stream) {
    const int nsb = (int)(K / kQK);
    GemmSet set = {};
    set.count = count;
    set.tile0[0] = 0;
    for (int p = 0; p < count; ++p) {
        set.w[p] = static_cast<const uint8_t *>(probs[p].w);
        set.y[p] = probs[p].y;
        set.N[p] = (int)probs[p].N;
        set.tile0[p + 1] = set.tile0[p] + (int)((probs[p].N + 127) / 128);   // WN = 128
    }
    const int64_t tiles_n = set.tile0[count];
    if (M > 64) {
        const int s = choose_splits(tiles_n, (M + 127) / 128, nsb, 128 * 128);
        return launch_tile<2, 2, 2>(set, nsb, codes, scales, sums, M, s, stream);
    }
    if (M > 32) {
        const int s = choose_splits(tiles_n, (M + 63) / 64, nsb, 128 * 64);
        return launch_tile<2, 1, 2>(set, nsb, codes, scales, sums, M, s, stream);
    }
    const int s = choose_splits(tiles_n, (M + 31) / 32, nsb, 128 * 32);
    return launch_tile<2, 1, 1>(set, nsb, codes, scales, sums, M, s, stream);
}

hipError_t launch_gemm(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       hipStream_t stream) {
    const GemmProblem p = {w, y, N};
    return launch_gemm_batch(&p, 1, K, codes, scales, sums, M, stream);
}

}  // namespace q4k
