// Prefill GEMM: y[M][N] = Q8(x)[M][K] * W^T with W in Q4_K, any M >= 1.
//
// Prefill is compute-bound ("genie-ai-runtime ...", section 3: batched
// layer-major prefill, Path E tensor-core kernel), so the contraction runs on
// the matrix cores.  With x^ = a*c (Q8: one fp32 scale a per 32 codes c) and
// w = d*sc[j]*q - dmin*mn[j] (Q4_K), one output is
//
//   y[m][n] = sum_b d[n,b] * sum_j a[m,b,j] * E[m,n,b,j]
//           - sum_b sum_j (dmin*mn)[n,b,j] * (a*S)[m,b,j],
//   E[m,n,b,j] = sum_{i<32} (sc*q)[n,b,j,i] * c[m,b,j,i]   (an integer),
//
// with S the code sum of one activation block.
//
// Main term.  Both matrix-core operands hold integers exactly in fp16: the
// weight operand sc*q <= 945 (made from the nibbles with one byte permute and
// one fused packed fp16 fma per pair: (1024 + q)*sc - 1024*sc), the activation
// operand the code c (a byte permute and one packed fp16 add per pair).  Two
// v_mfma_f32_32x32x16_f16 per 32x32 tile give E exactly (|E| < 2^22, every
// partial sum an integer below 2^24), which is sc * (the sub-block's integer
// dot).  The vector ALU then does one fma per output and sub-block,
// u = a*E + u, with a the same for all 16 outputs of a lane (a lane holds one
// activation row), and one fma per output and super-block, acc = d*u + acc.
//
// Min term.  Per super-block, sum_j (-dmin*mn_j) * (a*S)_j is an 8-long
// contraction; both factors (fp32; -dmin*mn exactly, a*S rounded once) are
// split into three bf16 parts hi + mid + lo (each rounded to nearest from
// the remainder, so the parts sum to the value exactly) and the six products
// above 2^-24 relative (hh, hm, mh, hl, mm, lh) fill the 48 k-slots of three
// v_mfma_f32_32x32x16_bf16, accumulated straight into acc.
//
// An int8 contraction (v_mfma_i32_32x32x32_i8 on the raw nibbles) needs, per
// output and sub-block, an int-to-float convert, the product of the two
// per-32-element scales (one from the weight row, one from the activation
// row) and an fma: three vector ops where this layout needs one.
//
// Staging: a quarter super-block (64 elements of K: two sub-blocks, which
// share one 32-byte group of quant bytes) per step, double-buffered in LDS.
// The waves are specialised: on each SIMD one wave only reads operands from
// LDS and runs the matrix-core ops and their epilogue, and one only loads raw
// blocks from global memory and converts them into the other LDS buffer.  The
// raw data of a whole super-block is loaded in one burst, four to eight steps
// before its conversion.  One barrier per step.
// Workgroup tile (64*WVN) weight rows x (32*TM*WVM) activation rows, one
// matrix-core wave per 64 x 32*TM outputs.
//
// Work split (deterministic).  The work is a sequence of units, one per
// (tile, super-block); tile t = column-block * (M tiles) + M tile, so the M
// tiles of one weight column-block are adjacent.  Workgroup g takes units
// [g*U/G, (g+1)*U/G): whole tiles, plus at most a partial tile at each end.
// Workgroups are numbered so that the 8 XCDs hold contiguous unit ranges
// (blockIdx % 8 is the XCD), which keeps a column-block's weights in one L2.
// A whole tile is stored directly.  A partial tile is written to a slot of
// the workspace, and a per-(tile, wave) counter, incremented after a
// device-scope release fence, tells the last contributor to arrive; that one
// adds the parts in contributor order (so the bits do not depend on arrival
// order), writes y and returns the counter to zero.  Without a workspace the
// grid has one workgroup per tile and no partial tiles.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "q4k_internal.h"

// GEMM_I8 selects the int8 contraction (v_mfma_i32_32x32x32_i8 on the raw
// quants and codes, exact int32 sub-block dots, fp32 epilogue
// acc += D * (a * d*sc)) instead of the fp16 one on integer-valued operands.
// Both are parity-tested; on the 512-token prefill the int8 one measured
// about 1.3x slower (three vector ops per output and sub-block against one), so
// fp16 is the default.  The build links the int8 form into a second library
// (libq4k_gemm_int8.so) beside the default one.
#ifndef GEMM_I8
#define GEMM_I8 false
#endif

namespace q4k {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int NXCD = 8;
constexpr int TN = 2;        // 32-row weight tiles per matrix-core wave
constexpr int OSTR = 72;     // fp16 per operand row and step: [kh 2][s 2][lh 2][8] + 8 pad

constexpr int QSTR = 80;     // bytes per int8 operand row and step: [s 2][lh 2][16] + 16 pad
constexpr int kQ6SB = 210;   // bytes per Q6_K super-block

// fp16 operands: integer-valued sc*q and codes.
template <int WN, int WM>
struct __attribute__((aligned(16))) LdsF {
    _Float16 aw[2][WN][OSTR];          // sc*q of a step's two sub-blocks
    _Float16 bx[2][WM][OSTR];          // codes of a step's two sub-blocks
    float dn[2][WN];                   // d of the super-block (by super-block parity)
    float as[2][8][WM];                // activation block scale a[j][row]
    unsigned short wm[2][3][WN][8];    // -(dmin*mn_j) as bf16 hi, mid, lo
    unsigned short pm[2][3][WM][8];    // (a*S)_j as bf16 hi, mid, lo
};
// int8 operands: the 4-bit quants q and the codes as they are.
template <int WN, int WM>
struct __attribute__((aligned(16))) LdsI {
    uint8_t aq[2][WN][QSTR];           // q of a step's two sub-blocks
    int8_t bc[2][WM][QSTR];            // codes of a step's two sub-blocks
    float ws[2][8][WN];                // d*sc_j per weight row
    float as[2][8][WM];
    unsigned short wm[2][3][WN][8];
    unsigned short pm[2][3][WM][8];
};
// Q6_K fp16 operands: sc*(q - 32) of a 16-weight sub-block as two exact
// parts, 16*sc*(q_hi - 2) (q_hi the quant's top 2 bits) and sc*q_lo (its low
// 4 bits), and the codes.  No min term.
template <int WN, int WM>
struct __attribute__((aligned(16))) LdsQ6 {
    _Float16 aw[2][WN][OSTR];          // sc*q_lo of a step's two 32-blocks
    _Float16 ah[2][WN][OSTR];          // 16*sc*(q_hi - 2)
    _Float16 bx[2][WM][OSTR];          // codes
    float dn[2][WN];                   // d of the super-block (by super-block parity)
    float as[2][8][WM];                // activation block scale a[j][row]
};
template <int WN, int WM, bool I8, bool Q6>
using Lds = typename std::conditional<
    Q6, LdsQ6<WN, WM>,
    typename std::conditional<I8, LdsI<WN, WM>, LdsF<WN, WM>>::type>::type;

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

// Unit ranges of the workgroups and the split-tile workspace.
struct Sched {
    int64_t units;     // tiles * nsb
    int groups;        // G, workgroups in the grid
    int tiles_m;       // M tiles
    float *part;       // 2 partial-tile slots per workgroup (null: no partial tiles)
    int *cnt;          // one counter per (tile, matrix-core wave)
};

template <int WVN, int WVM, int TM, int NV>
struct Cfg {
    static constexpr int WN = 32 * TN * WVN;
    static constexpr int WM = 32 * TM * WVM;
    static constexpr int NC = WVN * WVM;           // matrix-core waves
    static constexpr int P = 64 * NV;              // converting lanes (NV converting waves)
    static constexpr int T = 64 * (NC + NV);
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
// bf16 bits of v rounded to nearest, ties to even (v finite).
__device__ __forceinline__ unsigned bf16_rn(float v) {
    const unsigned b = __float_as_uint(v);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
// v = hi + mid + lo exactly for any fp32 v (each part rounded to nearest
// from the remainder left by the parts before it).
__device__ __forceinline__ void split3(float v, unsigned &hi, unsigned &mid, unsigned &lo) {
    hi = bf16_rn(v);
    const float r1 = v - __uint_as_float(hi << 16);
    mid = bf16_rn(r1);
    const float r2 = r1 - __uint_as_float(mid << 16);
    lo = bf16_rn(r2);
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
// 6-bit scale (or min) of sub-block J from the header dwords.
template <int J>
__device__ __forceinline__ unsigned scale6(const u32x4 &h, bool min) {
    const unsigned lo = min ? h.z : h.y;
    if (J < 4) return (lo >> (8 * J)) & 63u;
    const int sh = 8 * (J - 4);
    return ((h.w >> (sh + (min ? 4 : 0))) & 15u) | (((lo >> (sh + 6)) & 3u) << 4);
}

// Workgroup -> unit range.  floor(g*U/G) is the first unit of workgroup g; the
// workgroup holding unit u is floor(((u+1)*G - 1)/U).
__device__ __forceinline__ int64_t range_begin(int64_t g, const Sched &s) {
    return g * s.units / s.groups;
}
__device__ __forceinline__ int64_t group_of(int64_t u, const Sched &s) {
    return ((u + 1) * s.groups - 1) / s.units;
}

struct Tile {
    const uint8_t *w;
    float *y;
    int N, n0, m0;
};

// Position in the unit sequence, advanced one unit at a time (no division
// in the loops): tile t = vt * tiles_m + mt, super-block b, and the tile's
// product, weight rows and activation rows.  The product is picked with a
// compile-time select chain over the batch, so its pointers stay in scalar
// registers.
template <int WN, int WM>
struct Walk {
    int t, b, vt, mt;
    Tile tl;

    __device__ __forceinline__ void geometry(const GemmSet &set) {
        const uint8_t *w = set.w[0];
        float *y = set.y[0];
        int N = set.N[0], base = 0;
#pragma unroll
        for (int k = 1; k < kMaxGemmBatch; ++k)
            if (k < set.count && vt >= set.tile0[k]) {
                w = set.w[k];
                y = set.y[k];
                N = set.N[k];
                base = set.tile0[k];
            }
        tl.w = w;
        tl.y = y;
        tl.N = N;
        tl.n0 = (vt - base) * WN;
        tl.m0 = mt * WM;
    }
    __device__ __forceinline__ void start(const GemmSet &set, int64_t u, int nsb, int tiles_m) {
        t = (int)(u / nsb);
        b = (int)(u - (int64_t)t * nsb);
        vt = t / tiles_m;
        mt = t - vt * tiles_m;
        geometry(set);
    }
    __device__ __forceinline__ void next(const GemmSet &set, int nsb, int tiles_m) {
        if (++b < nsb) return;
        b = 0;
        ++t;
        if (++mt == tiles_m) {
            mt = 0;
            ++vt;
        }
        geometry(set);
    }
};

template <int WVN, int WVM, int TM, int NV, bool I8, bool Q6>
__global__ __launch_bounds__(64 * (WVN * WVM + NV), 1) void gemm_kernel(
    const GemmSet set, const Sched sch, int nsb, const int8_t *__restrict__ codes,
    const float *__restrict__ scales, const int32_t *__restrict__ sums, int M) {
    using C = Cfg<WVN, WVM, TM, NV>;
    constexpr int WN = C::WN, WM = C::WM, P = C::P, NC = C::NC;
    extern __shared__ __attribute__((aligned(16))) uint8_t lds_raw[];
    Lds<WN, WM, I8, Q6> &L = *reinterpret_cast<Lds<WN, WM, I8, Q6> *>(lds_raw);
    static_assert(!(I8 && Q6), "the Q6_K contraction is the fp16 one");

    const int G = sch.groups;
    const int gi = (G % NXCD == 0) ? (int)(blockIdx.x % NXCD) * (G / NXCD) + (int)(blockIdx.x / NXCD)
                                   : (int)blockIdx.x;
    const int64_t ub = range_begin(gi, sch), ue = range_begin(gi + 1, sch);
    if (ub >= ue) return;   // the whole workgroup exits, before any barrier
    const int K = nsb * 256, nblk = nsb * 8;
    const int64_t row_bytes = (int64_t)nsb * (Q6 ? kQ6SB : 144);
    const int tid = threadIdx.x;

    if (tid >= 64 * NC) {
        // ---------------- converting waves ----------------
        const int p = tid - 64 * NC;
        // Raw loads.  Rows past N or M read row N-1 / M-1 and units past the
        // end of the range read its last unit (branch-free loads): they only
        // feed outputs or buffers that are never used.
        struct Step {                 // one step: quant bytes, activation codes
            u32x4 q[C::NA];
            i32x4 c0[C::NB], c1[C::NB];
        };
        struct Block {                // one super-block: headers, block scales and sums
            u32x4 h[C::NA];
            float a[C::NB][8];
            int s[C::NB][8];
        };
        // Two units' worth of raw data: register set 4k + g holds quarter g of
        // the unit in slot k.  A unit's weight bytes (the two lanes of a row
        // read its 144 bytes) and its activation bytes (256 codes per row,
        // block scales and sums) are each loaded in one burst, so every cache
        // line is read within a few instructions (loaded one quarter per step,
        // each line was fetched again for every quarter); it is converted one
        // and two units later.
        // Q6_K: a 210-byte super-block starts at an even byte, so each 16-byte
        // field the lane needs is read as 5 dwords from the 4-byte boundary at
        // or below it and shifted into place at conversion (every read stays
        // inside the super-block).  Fields of lane c of a row: ql[16c + 32i]
        // (i < 4), qh[16c + 32i] (i < 2), the 16 scales; d by a 2-byte load.
        struct Q6Raw {
            unsigned ql[4][5], qh[2][5], sc[5];
            unsigned d, odd;          // d's fp16 bits; 2 if the super-block starts at 2 mod 4
        };
        Step S[8];
        Block blk[2];
        Q6Raw q6[Q6 ? 2 : 1][C::NA];
        const bool vec_as = ((reinterpret_cast<uintptr_t>(scales) |
                              (Q6 ? 0 : reinterpret_cast<uintptr_t>(sums))) & 15) == 0;

        // The unit at pw into slot k, in two parts: its weight bytes
        // (load_w), then its activation bytes (load_a), after which pw moves
        // on (not past the last unit).
        Walk<WN, WM> pw;
        int64_t pu = ub;
        pw.start(set, ub, nsb, sch.tiles_m);
        auto load_w = [&](auto kc) {
            constexpr int k = decltype(kc)::value;
            const Tile &tl = pw.tl;
            const int b = pw.b;
#pragma unroll
            for (int i = 0; i < C::NA; ++i) {
                const int e = min(p + i * P, C::CA - 1);
                const int row = min(tl.n0 + (e >> 1), tl.N - 1);
                if constexpr (Q6) {
                    const uint8_t *sb = tl.w + (int64_t)row * row_bytes + (int64_t)b * kQ6SB;
                    const unsigned odd = (unsigned)(reinterpret_cast<uintptr_t>(sb) & 2);
                    const uint8_t *base = sb - odd;              // 4-byte aligned
                    const int c = e & 1;
                    // dword 4 of a field is only used when odd; otherwise dword 3 is
                    // read again (so no read passes the super-block's last byte)
                    auto field = [&](unsigned *r5, int o) {
                        const unsigned *q = reinterpret_cast<const unsigned *>(base + o);
                        r5[0] = q[0];
                        r5[1] = q[1];
                        r5[2] = q[2];
                        r5[3] = q[3];
                        r5[4] = q[odd ? 4 : 3];
                    };
                    Q6Raw &R = q6[Q6 ? k : 0][i];
#pragma unroll
                    for (int f = 0; f < 4; ++f) field(R.ql[f], 16 * c + 32 * f);
#pragma unroll
                    for (int f = 0; f < 2; ++f) field(R.qh[f], 128 + 16 * c + 32 * f);
                    field(R.sc, 192);
                    R.d = *reinterpret_cast<const unsigned short *>(sb + 208);
                    R.odd = odd;
                } else {
                    const uint8_t *src = tl.w + (int64_t)row * row_bytes + (int64_t)b * 144;
                    blk[k].h[i] = *reinterpret_cast<const u32x4 *>(src);
#pragma unroll
                    for (int g = 0; g < 4; ++g)
                        S[4 * k + g].q[i] = *reinterpret_cast<const u32x4 *>(src + 16 + 32 * g + 16 * (e & 1));
                }
            }
        };
        auto load_a = [&](auto kc) {
            constexpr int k = decltype(kc)::value;
            const Tile &tl = pw.tl;
            const int b = pw.b;
#pragma unroll
            for (int i = 0; i < C::NB; ++i) {
                const int e = min(p + i * P, C::CB - 1);
                const int row = min(tl.m0 + (e >> 1), M - 1);
                const int8_t *src = codes + (int64_t)row * K + 256 * b + 32 * (e & 1);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    S[4 * k + g].c0[i] = *reinterpret_cast<const i32x4 *>(src + 64 * g);
                    S[4 * k + g].c1[i] = *reinterpret_cast<const i32x4 *>(src + 64 * g + 16);
                }
                const int64_t o = (int64_t)row * nblk + 8 * b;
                if (vec_as) {
                    const f32x4 a0 = *reinterpret_cast<const f32x4 *>(scales + o);
                    const f32x4 a1 = *reinterpret_cast<const f32x4 *>(scales + o + 4);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        blk[k].a[i][j] = a0[j];
                        blk[k].a[i][4 + j] = a1[j];
                    }
                    if constexpr (!Q6) {
                        const i32x4 s0 = *reinterpret_cast<const i32x4 *>(sums + o);
                        const i32x4 s1 = *reinterpret_cast<const i32x4 *>(sums + o + 4);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            blk[k].s[i][j] = s0[j];
                            blk[k].s[i][4 + j] = s1[j];
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        blk[k].a[i][j] = scales[o + j];
                        if constexpr (!Q6) blk[k].s[i][j] = sums[o + j];
                    }
                }
            }
            if (pu + 1 < ue) {
                pw.next(set, nsb, sch.tiles_m);
                ++pu;
            }
        };

        // Step g of a super-block (raw step in a register set, super-block data
        // in B) -> LDS buffer F and super-block parity Q.  Lanes that share a
        // row write identical header values.
        auto convert = [&](auto kc, auto gc, auto bufc, int Q) {
            constexpr int k = decltype(kc)::value;
            constexpr int g = decltype(gc)::value;
            constexpr int F = decltype(bufc)::value;
            const Step &R = S[4 * k + g];
            const Block &B = blk[k];
            if constexpr (Q6) {
#pragma unroll
            for (int i = 0; i < C::NA; ++i) {
                const int e = p + i * P;
                if (C::CA % P != 0 && e >= C::CA) continue;
                const int row = e >> 1, c = e & 1;
                const Q6Raw &W = q6[k][i];
                const unsigned sh = W.odd;   // bytes to shift the 5-dword reads by
                auto field = [&](const unsigned *r5) {
                    u32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __builtin_amdgcn_alignbyte(r5[j + 1], r5[j], sh);
                    return v;
                };
                // step g: elements 64g + 16c + j (32-block 2g) and 64g + 32 + 16c + j
                // (block 2g + 1), j < 16: low 4 bits in ql[64h + 16c + j] and
                // ql[64h + 32 + 16c + j] (high nibble for odd g), high 2 bits in
                // qh[32h + 16c + j] bits 4(g%2) and 4(g%2) + 2; scales
                // sc[4g + c] and sc[4g + 2 + c]
                constexpr int h = g >> 1, od = g & 1;
                const u32x4 qa = field(W.ql[2 * h]), qb = field(W.ql[2 * h + 1]);
                const u32x4 qhv = field(W.qh[h]);
                const u32x4 scv = field(W.sc);
                u32x4 la, lb, ha, hb;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    la[j] = (od ? qa[j] >> 4 : qa[j]) & 0x0F0F0F0Fu;
                    lb[j] = (od ? qb[j] >> 4 : qb[j]) & 0x0F0F0F0Fu;
                    ha[j] = (qhv[j] >> (4 * od)) & 0x03030303u;
                    hb[j] = (qhv[j] >> (4 * od + 2)) & 0x03030303u;
                }
                auto sc_byte = [&](int idx) {   // int8 scale idx of the super-block
                    return (float)(int8_t)((scv[idx >> 2] >> (8 * (idx & 3))) & 0xFFu);
                };
                const float sa = c ? sc_byte(4 * g + 1) : sc_byte(4 * g);
                const float sb2 = c ? sc_byte(4 * g + 3) : sc_byte(4 * g + 2);
                const half2 m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
                const half2 m1026 = {(_Float16)-1026.0f, (_Float16)-1026.0f};
                const half2 va = {(_Float16)sa, (_Float16)sa}, vb = {(_Float16)sb2, (_Float16)sb2};
                const half2 wa = {(_Float16)(16.0f * sa), (_Float16)(16.0f * sa)};
                const half2 wb = {(_Float16)(16.0f * sb2), (_Float16)(16.0f * sb2)};
                // q_lo * sc: (1024 + q_lo) - 1024 is exact, and so is the product
                // (|sc * q_lo| <= 1920); 16 sc (q_hi - 2) likewise (a multiple of
                // 16 of magnitude <= 4096)
                auto lo8 = [&](unsigned v0, unsigned v1, half2 sv) {
                    return cat4((bias_pair_lo(v0) + m1024) * sv, (bias_pair_hi(v0) + m1024) * sv,
                                (bias_pair_lo(v1) + m1024) * sv, (bias_pair_hi(v1) + m1024) * sv);
                };
                auto hi8 = [&](unsigned v0, unsigned v1, half2 sv) {
                    return cat4((bias_pair_lo(v0) + m1026) * sv, (bias_pair_hi(v0) + m1026) * sv,
                                (bias_pair_lo(v1) + m1026) * sv, (bias_pair_hi(v1) + m1026) * sv);
                };
                _Float16 *dl = &L.aw[F][row][32 * c];
                _Float16 *dh = &L.ah[F][row][32 * c];
                *reinterpret_cast<half8 *>(dl + 0) = lo8(la.x, la.y, va);
                *reinterpret_cast<half8 *>(dl + 8) = lo8(la.z, la.w, va);
                *reinterpret_cast<half8 *>(dl + 16) = lo8(lb.x, lb.y, vb);
                *reinterpret_cast<half8 *>(dl + 24) = lo8(lb.z, lb.w, vb);
                *reinterpret_cast<half8 *>(dh + 0) = hi8(ha.x, ha.y, wa);
                *reinterpret_cast<half8 *>(dh + 8) = hi8(ha.z, ha.w, wa);
                *reinterpret_cast<half8 *>(dh + 16) = hi8(hb.x, hb.y, wb);
                *reinterpret_cast<half8 *>(dh + 24) = hi8(hb.z, hb.w, wb);
                if (g == 0 && c == 0)
                    L.dn[Q][row] = (float)__builtin_bit_cast(_Float16, (unsigned short)W.d);
            }
            } else {
#pragma unroll
            for (int i = 0; i < C::NA; ++i) {
                const int e = p + i * P;
                if (C::CA % P != 0 && e >= C::CA) continue;   // (no branch when the chunks tile the lanes)
                const int row = e >> 1, c = e & 1;
                const u32x4 h = B.h[i], q = R.q[i];
                // low nibbles: sub-block 2g, high nibbles: sub-block 2g+1; byte t
                // of the chunk is element 16c + t of both
                if constexpr (I8) {
                    u32x4 lo, hi;
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        lo[k] = q[k] & 0x0F0F0F0Fu;
                        hi[k] = (q[k] >> 4) & 0x0F0F0F0Fu;
                    }
                    // [s][lh = c][16]
                    *reinterpret_cast<u32x4 *>(&L.aq[F][row][16 * c]) = lo;
                    *reinterpret_cast<u32x4 *>(&L.aq[F][row][32 + 16 * c]) = hi;
                    if (g == 0) {
                        // lane c of the row: d*sc_j for j = 4c .. 4c+3
                        const float d = half_lo(h.x);
                        const float w0 = d * (float)(c ? scale6<4>(h, false) : scale6<0>(h, false));
                        const float w1 = d * (float)(c ? scale6<5>(h, false) : scale6<1>(h, false));
                        const float w2 = d * (float)(c ? scale6<6>(h, false) : scale6<2>(h, false));
                        const float w3 = d * (float)(c ? scale6<7>(h, false) : scale6<3>(h, false));
                        L.ws[Q][4 * c + 0][row] = w0;
                        L.ws[Q][4 * c + 1][row] = w1;
                        L.ws[Q][4 * c + 2][row] = w2;
                        L.ws[Q][4 * c + 3][row] = w3;
                    }
                } else {
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
                // [kh = c][s][lh][8]: the two lanes of a row land 16 banks apart
                _Float16 *dst = &L.aw[F][row][32 * c];
                *reinterpret_cast<half8 *>(dst + 0) = conv(lo.x, lo.y, sv0, bv0);
                *reinterpret_cast<half8 *>(dst + 8) = conv(lo.z, lo.w, sv0, bv0);
                *reinterpret_cast<half8 *>(dst + 16) = conv(hi.x, hi.y, sv1, bv1);
                *reinterpret_cast<half8 *>(dst + 24) = conv(hi.z, hi.w, sv1, bv1);
                if constexpr (!I8)
                    if (g == 0) L.dn[Q][row] = half_lo(h.x);
                }
                if (g == 0) {
                    // lane c of the row: the three parts of -dmin*mn_j for j = 4c .. 4c+3
                    const float dmin = half_hi(h.x);
                    const unsigned m4[4] = {c ? scale6<4>(h, true) : scale6<0>(h, true),
                                            c ? scale6<5>(h, true) : scale6<1>(h, true),
                                            c ? scale6<6>(h, true) : scale6<2>(h, true),
                                            c ? scale6<7>(h, true) : scale6<3>(h, true)};
                    unsigned pt[3][4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) split3(-dmin * (float)m4[k], pt[0][k], pt[1][k], pt[2][k]);
#pragma unroll
                    for (int part = 0; part < 3; ++part) {
                        const u32x2 pv = {pt[part][0] | (pt[part][1] << 16), pt[part][2] | (pt[part][3] << 16)};
                        *reinterpret_cast<u32x2 *>(&L.wm[Q][part][row][4 * c]) = pv;
                    }
                }
            }
            }
            const half2 m1152 = {(_Float16)-1152.0f, (_Float16)-1152.0f};
#pragma unroll
            for (int i = 0; i < C::NB; ++i) {
                const int e = p + i * P;
                if (C::CB % P != 0 && e >= C::CB) continue;
                const int row = e >> 1, s = e & 1;
                if constexpr (I8) {
                    // [s][lh][16]: elements 0..15 and 16..31 of sub-block s
                    *reinterpret_cast<i32x4 *>(&L.bc[F][row][32 * s]) = R.c0[i];
                    *reinterpret_cast<i32x4 *>(&L.bc[F][row][32 * s + 16]) = R.c1[i];
                } else {
                // 8 codes -> fp16 (c ^ 0x80 is c + 128 as a byte)
                auto conv = [&](unsigned v0, unsigned v1) {
                    const unsigned u0 = v0 ^ 0x80808080u, u1 = v1 ^ 0x80808080u;
                    return cat4(bias_pair_lo(u0) + m1152, bias_pair_hi(u0) + m1152,
                                bias_pair_lo(u1) + m1152, bias_pair_hi(u1) + m1152);
                };
                // sub-block s of the step, [kh][s][lh][8]
                _Float16 *dst = &L.bx[F][row][16 * s];
                const i32x4 c0 = R.c0[i], c1 = R.c1[i];
                *reinterpret_cast<half8 *>(dst + 0) = conv(c0.x, c0.y);    // elements 0..7
                *reinterpret_cast<half8 *>(dst + 8) = conv(c0.z, c0.w);    // 8..15
                *reinterpret_cast<half8 *>(dst + 32) = conv(c1.x, c1.y);   // 16..23
                *reinterpret_cast<half8 *>(dst + 40) = conv(c1.z, c1.w);   // 24..31
                }
                if constexpr (Q6) {
                    // lane s of the row: the scales of blocks 4s .. 4s+3
                    if (g == 0)
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            L.as[Q][4 * s + k][row] = s ? B.a[i][4 + k] : B.a[i][k];
                } else if (g == 0) {
                    // lane s of the row: the scales and min-term parts of blocks 4s .. 4s+3
                    unsigned pt[3][4];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float a = s ? B.a[i][4 + k] : B.a[i][k];
                        const int sj = s ? B.s[i][4 + k] : B.s[i][k];
                        L.as[Q][4 * s + k][row] = a;
                        split3(a * (float)sj, pt[0][k], pt[1][k], pt[2][k]);
                    }
#pragma unroll
                    for (int part = 0; part < 3; ++part) {
                        const unsigned lo2 = pt[part][0] | (pt[part][1] << 16);
                        const unsigned hi2 = pt[part][2] | (pt[part][3] << 16);
                        unsigned *dstp = reinterpret_cast<unsigned *>(&L.pm[Q][part][row][4 * s]);
                        dstp[0] = lo2;
                        dstp[1] = hi2;
                    }
                }
            }
        };

        // Per step: convert the next step into the other LDS buffer, barrier.
        // Units alternate between slots 0 and 1.  Per unit: convert quarters
        // 1..3 of it and quarter 0 of the next unit, one per step (the
        // matrix-core waves read the LDS buffer a step later).  Once its last
        // quarter is converted, the slot's weight registers are reloaded with
        // the unit two ahead, and its activation registers a step later, at
        // the step where the matrix-core waves end a super-block: issuing the
        // whole reload at once made that one step of four the converting
        // waves' slowest while the matrix-core waves' slowest came a step
        // later (the 36-layer M = 512 step: 244 -> 230 us per layer).
        __builtin_amdgcn_s_setprio(2);   // conversion feeds the next step: issue it first
        load_w(IC<0>{});
        load_a(IC<0>{});
        load_w(IC<1>{});
        load_a(IC<1>{});
        convert(IC<0>{}, IC<0>{}, IC<0>{}, 0);
        __syncthreads();
#pragma unroll 1
        for (int64_t u = ub; u < ue; u += 2) {
            convert(IC<0>{}, IC<1>{}, IC<1>{}, 0);
            __syncthreads();
            convert(IC<0>{}, IC<2>{}, IC<0>{}, 0);
            __syncthreads();
            convert(IC<0>{}, IC<3>{}, IC<1>{}, 0);
            load_w(IC<0>{});
            __syncthreads();
            convert(IC<1>{}, IC<0>{}, IC<0>{}, 1);
            load_a(IC<0>{});
            __syncthreads();
            if (u + 1 >= ue) break;
            convert(IC<1>{}, IC<1>{}, IC<1>{}, 1);
            __syncthreads();
            convert(IC<1>{}, IC<2>{}, IC<0>{}, 1);
            __syncthreads();
            convert(IC<1>{}, IC<3>{}, IC<1>{}, 1);
            load_w(IC<1>{});
            __syncthreads();
            convert(IC<0>{}, IC<0>{}, IC<0>{}, 0);
            load_a(IC<1>{});
            __syncthreads();
        }
        return;
    }

    // ---------------- matrix-core waves ----------------
    const int lane = tid & 63, wave = tid >> 6;
    const int wn = wave / WVM, wm = wave % WVM;
    const int lr = lane & 31, lh = lane >> 5;

    f32x16 acc[TN][TM], usb[TN][TM];
    const f32x16 zero16 = {};

    // Sub-block J of the super-block (sub-block s of the step in LDS buffer F).
    // fp16: two matrix-core ops per 32x32 tile give E; u = a*E (+ u).
    // int8: one gives the integer dot D; acc += D * (a * d*sc_J).
    auto compute = [&](auto bufc, auto sc, auto jc, int Q) {
        constexpr int F = decltype(bufc)::value;
        constexpr int s = decltype(sc)::value;
        constexpr int J = decltype(jc)::value;
        float a[TM];
#pragma unroll
        for (int t = 0; t < TM; ++t) a[t] = L.as[Q][J][(wm * TM + t) * 32 + lr];
        if constexpr (I8) {
            i32x4 A[TN], B[TM];
            float w[TN][16];
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const int r0 = (wn * TN + u) * 32;
                A[u] = *reinterpret_cast<const i32x4 *>(&L.aq[F][r0 + lr][32 * s + 16 * lh]);
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 w4 = *reinterpret_cast<const f32x4 *>(&L.ws[Q][J][r0 + 8 * q + 4 * lh]);
#pragma unroll
                    for (int k = 0; k < 4; ++k) w[u][4 * q + k] = w4[k];
                }
            }
#pragma unroll
            for (int t = 0; t < TM; ++t)
                B[t] = *reinterpret_cast<const i32x4 *>(&L.bc[F][(wm * TM + t) * 32 + lr][32 * s + 16 * lh]);
            const i32x16 zi = {};
#pragma unroll
            for (int u = 0; u < TN; ++u)
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    const i32x16 D = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[u], B[t], zi, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        acc[u][t][i] = fmaf((float)D[i], a[t] * w[u][i], acc[u][t][i]);
                }
        } else if constexpr (Q6) {
            // 4 matrix-core ops per 32x32 tile: elements 0..15 (high part, low
            // part), then 16..31; E = sum of sc*(q - 32)*code over the block
            half8 AH[TN][2], AL[TN][2], B[TM][2];
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const _Float16 *sl = &L.aw[F][(wn * TN + u) * 32 + lr][16 * s + 8 * lh];
                const _Float16 *sh = &L.ah[F][(wn * TN + u) * 32 + lr][16 * s + 8 * lh];
                AL[u][0] = *reinterpret_cast<const half8 *>(sl);
                AL[u][1] = *reinterpret_cast<const half8 *>(sl + 32);
                AH[u][0] = *reinterpret_cast<const half8 *>(sh);
                AH[u][1] = *reinterpret_cast<const half8 *>(sh + 32);
            }
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const _Float16 *src = &L.bx[F][(wm * TM + t) * 32 + lr][16 * s + 8 * lh];
                B[t][0] = *reinterpret_cast<const half8 *>(src);
                B[t][1] = *reinterpret_cast<const half8 *>(src + 32);
            }
#pragma unroll
            for (int u = 0; u < TN; ++u)
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    f32x16 e = __builtin_amdgcn_mfma_f32_32x32x16_f16(AH[u][0], B[t][0], zero16, 0, 0, 0);
                    e = __builtin_amdgcn_mfma_f32_32x32x16_f16(AL[u][0], B[t][0], e, 0, 0, 0);
                    e = __builtin_amdgcn_mfma_f32_32x32x16_f16(AH[u][1], B[t][1], e, 0, 0, 0);
                    e = __builtin_amdgcn_mfma_f32_32x32x16_f16(AL[u][1], B[t][1], e, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        usb[u][t][i] = J == 0 ? e[i] * a[t] : fmaf(e[i], a[t], usb[u][t][i]);
                }
        } else {
            half8 A[TN][2], B[TM][2];
#pragma unroll
            for (int u = 0; u < TN; ++u) {
                const _Float16 *src = &L.aw[F][(wn * TN + u) * 32 + lr][16 * s + 8 * lh];
                A[u][0] = *reinterpret_cast<const half8 *>(src);
                A[u][1] = *reinterpret_cast<const half8 *>(src + 32);
            }
#pragma unroll
            for (int t = 0; t < TM; ++t) {
                const _Float16 *src = &L.bx[F][(wm * TM + t) * 32 + lr][16 * s + 8 * lh];
                B[t][0] = *reinterpret_cast<const half8 *>(src);
                B[t][1] = *reinterpret_cast<const half8 *>(src + 32);
            }
#pragma unroll
            for (int u = 0; u < TN; ++u)
#pragma unroll
                for (int t = 0; t < TM; ++t) {
                    f32x16 e = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[u][0], B[t][0], zero16, 0, 0, 0);
                    e = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[u][1], B[t][1], e, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        usb[u][t][i] = J == 0 ? e[i] * a[t] : fmaf(e[i], a[t], usb[u][t][i]);
                }
        }
    };

    // End of a super-block: acc += d * u, then the min term on the matrix
    // cores.  A lane's outputs share one activation row m and span 16 weight
    // rows n (their d).
    constexpr int WP[6] = {0, 0, 1, 0, 1, 2};   // weight part of k-slot group 2p + lh
    constexpr int AP[6] = {0, 1, 0, 2, 1, 0};   // activation part
    auto finish = [&](int Q) {
#pragma unroll
        for (int u = 0; u < TN * !I8; ++u) {
            const int r0 = (wn * TN + u) * 32;
            float dv[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                f32x4 d4 = {};
                if constexpr (!I8) d4 = *reinterpret_cast<const f32x4 *>(&L.dn[Q][r0 + 8 * q + 4 * lh]);
#pragma unroll
                for (int k = 0; k < 4; ++k) dv[4 * q + k] = d4[k];
            }
#pragma unroll
            for (int t = 0; t < TM; ++t)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[u][t][i] = fmaf(dv[i], usb[u][t][i], acc[u][t][i]);
        }
        if constexpr (!Q6) {
#pragma unroll
        for (int pp = 0; pp < 3; ++pp) {
            bf16x8 W[TN], X[TM];
            const int wp = lh ? WP[2 * pp + 1] : WP[2 * pp];
            const int ap = lh ? AP[2 * pp + 1] : AP[2 * pp];
#pragma unroll
            for (int u = 0; u < TN; ++u)
                W[u] = *reinterpret_cast<const bf16x8 *>(&L.wm[Q][wp][(wn * TN + u) * 32 + lr][0]);
#pragma unroll
            for (int t = 0; t < TM; ++t)
                X[t] = *reinterpret_cast<const bf16x8 *>(&L.pm[Q][ap][(wm * TM + t) * 32 + lr][0]);
#pragma unroll
            for (int u = 0; u < TN; ++u)
#pragma unroll
                for (int t = 0; t < TM; ++t)
                    acc[u][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(W[u], X[t], acc[u][t], 0, 0, 0);
        }
        }
    };

    // Output of the lane for tile (u, t): activation row m, weight rows
    // n .. n+3 for each quarter q (n = n0 + ... + 8q + 4lh).
    auto store_y = [&](const Tile &tl) {
#pragma unroll
        for (int t = 0; t < TM; ++t) {
            const int m = tl.m0 + (wm * TM + t) * 32 + lr;
            if (m >= M) continue;
            float *yr = tl.y + (int64_t)m * tl.N;
            const bool vec = ((tl.N & 3) == 0) && ((reinterpret_cast<uintptr_t>(tl.y) & 15) == 0);
#pragma unroll
            for (int u = 0; u < TN; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = tl.n0 + (wn * TN + u) * 32 + 8 * q + 4 * lh;
                    const f32x4 v = {acc[u][t][4 * q], acc[u][t][4 * q + 1], acc[u][t][4 * q + 2],
                                     acc[u][t][4 * q + 3]};
                    if (vec && n + 3 < tl.N) {
                        *reinterpret_cast<f32x4 *>(yr + n) = v;
                    } else {
#pragma unroll
                        for (int k = 0; k < 4; ++k)
                            if (n + k < tl.N) yr[n + k] = v[k];
                    }
                }
        }
    };

    // Partial-tile slot layout: [wave][u][t][pair q][lane] float pairs.
    auto slot_ptr = [&](int64_t slot) {
        return sch.part + slot * (int64_t)(WN * WM) + (int64_t)wave * (TN * TM * 16 * 64);
    };

    // End of the unit range's part of tile t (units [s0, s1) of it).
    auto finish_tile = [&](const Walk<WN, WM> &w, int64_t s0, int64_t s1) {
        const int t = w.t;
        const Tile &tl = w.tl;
        const int64_t t0 = (int64_t)t * nsb, t1 = t0 + nsb;
        if (s0 == t0 && s1 == t1) {   // the whole tile
            store_y(tl);
            return;
        }
        const int64_t first = group_of(t0, sch), last = group_of(t1 - 1, sch);
        const int nparts = (int)(last - first + 1);
        // slot 0 of a workgroup: a tile that began before its range; slot 1:
        // the tile its range ends in
        const int64_t my_slot = 2 * (int64_t)gi + (s0 > t0 ? 0 : 1);
        // Parts go through agent-coherent accesses (relaxed atomic stores and
        // loads at agent scope), and the counter is only incremented once
        // every store of the wave has completed.  An agent-scope fence instead
        // would write back and invalidate the whole L2 of the XCD, evicting
        // the weight and activation tiles of every workgroup on it.
        unsigned long long *dst = reinterpret_cast<unsigned long long *>(slot_ptr(my_slot));
#pragma unroll
        for (int u = 0; u < TN; ++u)
#pragma unroll
            for (int tt = 0; tt < TM; ++tt)
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const unsigned long long v =
                        (unsigned long long)__float_as_uint(acc[u][tt][2 * q]) |
                        ((unsigned long long)__float_as_uint(acc[u][tt][2 * q + 1]) << 32);
                    __hip_atomic_store(dst + ((u * TM + tt) * 8 + q) * 64 + lane, v, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                }
        __builtin_amdgcn_s_waitcnt(0);   // every store above has completed
        int *cp = sch.cnt + (int64_t)t * NC + wave;
        int old = 0;
        if (lane == 0) old = __hip_atomic_fetch_add(cp, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        old = __shfl(old, 0);
        if (old != nparts - 1) return;
        // the last to arrive adds the parts in contributor order
        f32x16 sum[TN][TM];
        for (int k = 0; k < nparts; ++k) {
            const int64_t g2 = first + k;
            if (g2 == gi) {
#pragma unroll
                for (int u = 0; u < TN; ++u)
#pragma unroll
                    for (int tt = 0; tt < TM; ++tt) sum[u][tt] = k == 0 ? acc[u][tt] : sum[u][tt] + acc[u][tt];
                continue;
            }
            unsigned long long *src = reinterpret_cast<unsigned long long *>(
                slot_ptr(2 * g2 + (range_begin(g2, sch) > t0 ? 0 : 1)));
#pragma unroll
            for (int u = 0; u < TN; ++u)
#pragma unroll
                for (int tt = 0; tt < TM; ++tt)
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const unsigned long long v = __hip_atomic_load(
                            src + ((u * TM + tt) * 8 + q) * 64 + lane, __ATOMIC_RELAXED,
                            __HIP_MEMORY_SCOPE_AGENT);
                        const float x0 = __uint_as_float((unsigned)v);
                        const float x1 = __uint_as_float((unsigned)(v >> 32));
                        sum[u][tt][2 * q] = k == 0 ? x0 : sum[u][tt][2 * q] + x0;
                        sum[u][tt][2 * q + 1] = k == 0 ? x1 : sum[u][tt][2 * q + 1] + x1;
                    }
        }
#pragma unroll
        for (int u = 0; u < TN; ++u)
#pragma unroll
            for (int tt = 0; tt < TM; ++tt) acc[u][tt] = sum[u][tt];
        store_y(tl);
        if (lane == 0) __hip_atomic_store(cp, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    __syncthreads();
    Walk<WN, WM> at;
    at.start(set, ub, nsb, sch.tiles_m);
    int64_t seg0 = ub;   // first unit of the current tile segment
#pragma unroll
    for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b) acc[a][b] = zero16;
#pragma unroll 1
    for (int64_t u = ub; u < ue; ++u) {
        const int Q = (int)(u - ub) & 1;
        compute(IC<0>{}, IC<0>{}, IC<0>{}, Q);
        compute(IC<0>{}, IC<1>{}, IC<1>{}, Q);
        __syncthreads();
        compute(IC<1>{}, IC<0>{}, IC<2>{}, Q);
        compute(IC<1>{}, IC<1>{}, IC<3>{}, Q);
        __syncthreads();
        compute(IC<0>{}, IC<0>{}, IC<4>{}, Q);
        compute(IC<0>{}, IC<1>{}, IC<5>{}, Q);
        __syncthreads();
        compute(IC<1>{}, IC<0>{}, IC<6>{}, Q);
        compute(IC<1>{}, IC<1>{}, IC<7>{}, Q);
        finish(Q);
        if (u + 1 == ue || at.b + 1 == nsb) {
            finish_tile(at, seg0, u + 1);
            seg0 = u + 1;
#pragma unroll
            for (int a = 0; a < TN; ++a)
#pragma unroll
                for (int b = 0; b < TM; ++b) acc[a][b] = zero16;
        }
        at.next(set, nsb, sch.tiles_m);
        __syncthreads();
    }
}

template <int WVN, int WVM, int TM, int NV, bool I8 = GEMM_I8, bool Q6 = false>
hipError_t launch_tile(const GemmSet &set, int nsb, const int8_t *codes, const float *scales,
                       const int32_t *sums, int64_t M, void *ws, hipStream_t stream) {
    using C = Cfg<WVN, WVM, TM, NV>;
    const int64_t tiles_m = (M + C::WM - 1) / C::WM;
    const int64_t tiles = (int64_t)set.tile0[set.count] * tiles_m;
    Sched s = {};
    s.tiles_m = (int)tiles_m;
    s.units = tiles * nsb;
    s.groups = (int)tiles;
    const int64_t cus = std::min<int64_t>(cu_count(), kGemmMaxGroups);
    // Split tiles across workgroups only where whole tiles would leave CUs idle
    // in the last round, and only where the counters fit the workspace.  The
    // units are cut into one equal range per CU, except where cutting every
    // tile into the same whole number of parts still keeps at least 90 % of
    // the CUs busy (80 tiles: 3 parts on 240 workgroups): then no range
    // straddles two tiles and each tile has the fewest parts to add (the
    // 36-layer M = 512 step: {down} 56.7 -> 54.8 us, {o} 31.7 -> 31.3).
    if (ws && tiles % cus != 0 && tiles * C::NC <= kGemmCounters && s.units >= cus) {
        const int64_t whole = tiles < cus ? tiles * (cus / tiles) : 0;
        s.groups = (int)(10 * whole >= 9 * cus ? whole : cus);
        s.cnt = static_cast<int *>(ws);
        s.part = reinterpret_cast<float *>(static_cast<uint8_t *>(ws) + kGemmCounters * 4);
    }
    hipLaunchKernelGGL((gemm_kernel<WVN, WVM, TM, NV, I8, Q6>), dim3((unsigned)s.groups),
                       dim3(C::T), sizeof(Lds<C::WN, C::WM, I8, Q6>), stream, set, s, nsb, codes,
                       scales, sums, (int)M);
    return hipGetLastError();
}

// Clears the split-tile counters of a workspace.
__global__ __launch_bounds__(256) void clear_counters_kernel(int *cnt) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < kGemmCounters) cnt[i] = 0;
}

// Scratch of the allocation-free entry point: the split-tile counters and
// partial tiles of one GEMM launch, the same layout as a caller workspace.
constexpr size_t kScratchBytes = (size_t)kGemmCounters * 4 + (size_t)2 * kGemmMaxGroups * 128 * 128 * 4;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

}  // namespace

// Device address of `scratch` on the current device, looked up once per
// device (each device holds its own copy of the array); null if the runtime
// cannot resolve it.  The host-side name `scratch` is not a device address
// and is never passed to a kernel.
void *gemm_static_scratch() {
    static std::atomic<void *> ptr[64];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    void *p = ptr[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
        void *q = nullptr;
        if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
        ptr[dev].store(q, std::memory_order_release);
        p = q;
    }
    return p;
}

size_t gemm_static_scratch_bytes() { return kScratchBytes; }

hipError_t launch_clear_counters(void *workspace, hipStream_t stream) {
    hipLaunchKernelGGL(clear_counters_kernel, dim3((kGemmCounters + 255) / 256), dim3(256), 0,
                       stream, static_cast<int *>(workspace));
    return hipGetLastError();
}

size_t gemm_workspace_bytes() {
    return (size_t)kGemmCounters * 4 + (size_t)2 * kGemmMaxGroups * 128 * 128 * 4;
}

namespace {
GemmSet make_set(const GemmProblem *probs, int count) {
    GemmSet set = {};
    set.count = count;
    set.tile0[0] = 0;
    for (int p = 0; p < count; ++p) {
        set.w[p] = static_cast<const uint8_t *>(probs[p].w);
        set.y[p] = probs[p].y;
        set.N[p] = (int)probs[p].N;
        set.tile0[p + 1] = set.tile0[p] + (int)((probs[p].N + 127) / 128);   // WN = 128
    }
    return set;
}
}  // namespace

#ifndef GEMM_BIG
#define GEMM_BIG 2, 2, 2, 4
#endif

hipError_t launch_gemm_batch(const GemmProblem *probs, int count, int64_t K,
                             const int8_t *codes, const float *scales, const int32_t *sums,
                             int64_t M, void *workspace, hipStream_t stream) {
    // A few rows would leave the matrix-core tiles mostly idle: up to 8 rows
    // run q4k_gemv's kernels (the same bits), all products in one launch --
    // the matrix-core GEMV where it is preferred for the launch's rows, else
    // the streaming one.
    if (M <= 8 && stream_fits(M, K)) {
        GemvProblem gp[kMaxGemmBatch];
        int64_t rows = 0;
        for (int p = 0; p < count; ++p) {
            gp[p] = {probs[p].w, nullptr, probs[p].y, probs[p].N};
            rows += probs[p].N;
        }
        if (gemv_mfma_preferred(rows, K, M, scales, sums))
            return launch_gemv_mfma_batch(gp, count, K, codes, scales, sums, M, stream);
        return launch_gemv_batch_prepared(gp, count, K, codes, scales, sums, M, stream);
    }
    const int nsb = (int)(K / kQK);
    const GemmSet set = make_set(probs, count);
    if (M > 64) return launch_tile<GEMM_BIG>(set, nsb, codes, scales, sums, M, workspace, stream);
    if (M > 32) return launch_tile<2, 2, 1, 4>(set, nsb, codes, scales, sums, M, workspace, stream);
    return launch_tile<2, 1, 1, 2>(set, nsb, codes, scales, sums, M, workspace, stream);
}

// Q6_K weights: the same tiles, units and split, the fp16 contraction.
hipError_t launch_q6k_gemm_batch(const GemmProblem *probs, int count, int64_t K,
                                 const int8_t *codes, const float *scales, int64_t M,
                                 void *workspace, hipStream_t stream) {
    const int nsb = (int)(K / kQK);
    const GemmSet set = make_set(probs, count);
    if (M > 64)
        return launch_tile<2, 2, 2, 4, false, true>(set, nsb, codes, scales, nullptr, M, workspace,
                                                    stream);
    if (M > 32)
        return launch_tile<2, 2, 1, 4, false, true>(set, nsb, codes, scales, nullptr, M, workspace,
                                                    stream);
    return launch_tile<2, 1, 1, 2, false, true>(set, nsb, codes, scales, nullptr, M, workspace,
                                                stream);
}

hipError_t launch_gemm(const uint8_t *w, int64_t N, int64_t K, const int8_t *codes,
                       const float *scales, const int32_t *sums, int64_t M, float *y,
                       void *workspace, hipStream_t stream) {
    const GemmProblem p = {w, y, N};
    return launch_gemm_batch(&p, 1, K, codes, scales, sums, M, workspace, stream);
}

}  // namespace q4k
