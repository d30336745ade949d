// Device helpers shared by the GEMV-style kernels (decode GEMV and the
// routed-expert grouped GEMV).
//
// Lane <-> 16-byte quant chunk mapping: 8 lanes take one 144-byte super-block,
// lane l holding quant chunk l.  Chunk l holds, for g = l/2 and h = l%2,
// elements 64g+16h+i (low nibbles, sub-block 2g) and 64g+32+16h+i (high
// nibbles, sub-block 2g+1), i < 16.  After the partner exchange lane l owns the
// exact integer dot of sub-block j = l.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4k {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kQuadSwap1 = 0xB1;      // DPP quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // DPP quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // DPP lane i <-> 7-i within each 8 lanes

// DPP move within a lane quad or an 8-lane row half: every source lane
// exists, so no fallback value is needed.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}

// Sum over the 8 lanes of each aligned lane group.
__device__ __forceinline__ float group8_sum(float v) {
    v += dpp_f<kQuadSwap1>(v);
    v += dpp_f<kQuadSwap2>(v);
    v += dpp_f<kRowHalfMirror>(v);
    return v;
}

// The per-sub-block factor f_j = d*sc_j*D_j - dmin*mn_j*S_j of the epilogue
// a_j * f_j, with the mins product rounded on its own: fma(ds, D, -RN(dm*S)).
__device__ __forceinline__ float subblock_factor(float ds, int D, float dm, float S) {
#pragma clang fp contract(off)
    return fmaf(ds, (float)D, -(dm * S));
}

// Super-block term of one weight row and activation row: the sum over a lane
// group of e_j = a_j * f_j, lane l holding sub-block j = l, in one fixed order:
//   T = (u0 + u2) + (u7 + u5),   u_j = fma(a_j, f_j, RN(a_k * f_k)), k = j ^ 1.
// Lane 0 of the group returns T.  Written out (no contraction left to the
// compiler) because the matrix-core small-batch GEMV forms the same T from
// lanes laid out differently and must match it bit for bit.
__device__ __forceinline__ float superblock_term(float a, float f) {
#pragma clang fp contract(off)
    const float p = a * f;
    float v = fmaf(a, f, dpp_f<kQuadSwap1>(p));
    v = v + dpp_f<kQuadSwap2>(v);
    return v + dpp_f<kRowHalfMirror>(v);
}

// Q8 quantization of one block of 32 fp32 values held by an aligned group of
// 8 lanes, 4 consecutive values per lane (lane i of the group: values
// 4i..4i+3).  Scale d = fl32(amax / 127); code = rne(fl32(x / d)); an
// all-zero block has d = 0 and codes 0 (the Q8 activation format of q4k.h).
// Every division is correctly rounded, so the codes are the IEEE ones bit
// for bit:
//  * amax / 127: with y = RN(1/127), one correction step
//    q0 + RN(amax - 127 q0) * y is correctly rounded for every fp32 amax
//    (checked over all mantissas and exponents);
//  * x / d: the hardware division sequence without its range scaling -- the
//    reciprocal refined once, the quotient corrected twice.  For d in
//    [2^-100, 2^122) every intermediate stays normal when |x / d| >= 1/2
//    (smaller quotients give code 0 whatever their last bit); scales below
//    2^-100 take IEEE division instead (a wave-uniform branch, never taken for
//    ordinary activations).
// Rounding: adding 1.5 * 2^23 leaves rne(q) in two's complement in the low
// mantissa bits.  The fast branch needs no clamp: with d normal, |x| <= amax
// and d >= (amax / 127)(1 - 2^-24) bound |q| by 127 + 2^-17, so codes lie in
// [-127, 127].  A subnormal d carries fewer significant bits (amax / d can
// exceed 127.5), so the IEEE branch clamps.
// Returns this lane's 4 codes (value 4i+k in byte k); d and the block's code
// sum are the same on all 8 lanes.
struct Q8Lane {
    unsigned codes;
    float d;
    int sum;
};

// fl32(amax / 127), correctly rounded: with y = RN(1/127), one correction step
// q0 + RN(amax - 127 q0) * y.
__device__ __forceinline__ float q8_scale(float amax) {
    constexpr float y = 1.0f / 127.0f;
    const float q0 = amax * y;
    return __builtin_fmaf(__builtin_fmaf(-127.0f, q0, amax), y, q0);
}

// The reciprocal of d refined once, for q8_quotient.
__device__ __forceinline__ float q8_recip(float d) {
    const float r0 = __builtin_amdgcn_rcpf(d);
    return __builtin_fmaf(__builtin_fmaf(-d, r0, 1.0f), r0, r0);
}

// RN(x / d) for d in [2^-100, 2^122) and |x / d| >= 1/2 (smaller quotients
// round to code 0 whatever their last bit): the quotient x * r1 corrected twice.
__device__ __forceinline__ float q8_quotient(float x, float d, float r1) {
    float t = x * r1;
    t = __builtin_fmaf(__builtin_fmaf(-d, t, x), r1, t);
    return __builtin_fmaf(__builtin_fmaf(-d, t, x), r1, t);
}
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ Q8Lane quantize_block8(f32x4 v) {
    // |x| compared as unsigned bit patterns: the same order for non-negative floats
    unsigned a = max(max(__float_as_uint(v[0]) & 0x7FFFFFFFu, __float_as_uint(v[1]) & 0x7FFFFFFFu),
                     max(__float_as_uint(v[2]) & 0x7FFFFFFFu, __float_as_uint(v[3]) & 0x7FFFFFFFu));
    a = max(a, (unsigned)dpp_i<kQuadSwap1>((int)a));
    a = max(a, (unsigned)dpp_i<kQuadSwap2>((int)a));
    a = max(a, (unsigned)dpp_i<kRowHalfMirror>((int)a));
    const float amax = __uint_as_float(a);
    const float d = q8_scale(amax);
    const float dd = d == 0.0f ? 1.0f : d;   // all-zero block: +-0 / 1 gives code 0
    float q[4];
    if (__builtin_amdgcn_ballot_w64(dd < 0x1p-100f) != 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = __builtin_amdgcn_fmed3f(v[k] / dd, -127.0f, 127.0f);
    } else {
        const float r1 = q8_recip(dd);
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = q8_quotient(v[k], dd, r1);
    }
    unsigned b[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) b[k] = __float_as_uint(q[k] + 0x1.8p23f);
    Q8Lane r;
    const unsigned lo = __builtin_amdgcn_perm(b[1], b[0], 0x0c0c0400u);   // bytes: b0, b1
    const unsigned hi = __builtin_amdgcn_perm(b[3], b[2], 0x0c0c0400u);   // bytes: b2, b3
    r.codes = __builtin_amdgcn_perm(hi, lo, 0x05040100u);
    int sum = (int)(b[0] + b[1] + b[2] + b[3] - 4u * 0x4B400000u);
    sum += dpp_i<kQuadSwap1>(sum);
    sum += dpp_i<kQuadSwap2>(sum);
    sum += dpp_i<kRowHalfMirror>(sum);
    r.d = d;
    r.sum = sum;
    return r;
}

// SwiGLU of four values, h = silu(g) * u = g / (1 + e^-g) * u, evaluated in
// fp64 from the fp32 g, u and rounded to fp32 once (the expert FFN's
// nonlinearity; the same arithmetic wherever h is formed).
__device__ __forceinline__ float swiglu1(float g, float u) {
    const double gd = (double)g;
    return (float)(gd / (1.0 + exp(-gd)) * (double)u);
}
__device__ __forceinline__ f32x4 swiglu4(f32x4 g, f32x4 u) {
    f32x4 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = swiglu1(g[i], u[i]);
    return h;
}

// 16 bytes of weights, a plain (temporal) load: on MI355X the 36-layer decode
// step ran 0.793 ms with plain weight loads against 0.808 ms with loads marked
// non-temporal, and the routed-expert layer 2-8 % faster.
__device__ __forceinline__ u32x4 load_weights16(const uint8_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ float half_lo(unsigned v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v & 0xFFFF));
}
__device__ __forceinline__ float half_hi(unsigned v) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(v >> 16));
}

// Per-lane constants of the chunk mapping for lane l (0..7) of a group.
struct LaneMap {
    int l, g, h;
    int sh;        // 8 * (j & 3) for sub-block j = l
    bool lo4;      // j < 4
    int offA, offB;  // code offsets (within the super-block) paired with low / high nibbles
    __device__ explicit LaneMap(int lane_in_group) {
        l = lane_in_group;
        g = l >> 1;
        h = l & 1;
        sh = 8 * (l & 3);
        lo4 = l < 4;
        offA = 64 * g + 16 * h;
        offB = 64 * g + 32 + 16 * h;
    }
};

// Decode d*sc[j] and dmin*mn[j] for sub-block j = l from a super-block header.
__device__ __forceinline__ void decode_scale(const LaneMap &L, u32x4 hd, float &ds, float &dm) {
    const unsigned h1 = hd.y, h2 = hd.z, h3 = hd.w;
    unsigned sc, mn;
    if (L.lo4) {
        sc = (h1 >> L.sh) & 63u;
        mn = (h2 >> L.sh) & 63u;
    } else {
        sc = ((h3 >> L.sh) & 15u) | (((h1 >> (L.sh + 6)) & 3u) << 4);
        mn = ((h3 >> (L.sh + 4)) & 15u) | (((h2 >> (L.sh + 6)) & 3u) << 4);
    }
    ds = half_lo(hd.x) * (float)sc;
    dm = half_hi(hd.x) * (float)mn;
}

// The four dwords held by the lanes of this lane's quad (lane 4k+i holds
// dword i), as one vector.
__device__ __forceinline__ u32x4 quad_gather(unsigned v) {
    u32x4 h;
    h.x = (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, true);  // [0,0,0,0]
    h.y = (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, true);  // [1,1,1,1]
    h.z = (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, true);  // [2,2,2,2]
    h.w = (unsigned)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, true);  // [3,3,3,3]
    return h;
}

// d*sc_j and dmin*mn_j of sub-block j = lane l of the group, branch-free.
// With sh = 8*(j & 3) the 6-bit value is 4 bits of X at xs plus 2 bits of Y at
// ys: sc takes X = h1 (j < 4) or h3 (j >= 4) and Y = h1; mn takes X = h2 or
// h3 and Y = h2; xs = sh (+4 for mn when j >= 4); ys = sh+4 (j < 4) or sh+6
// -- the header's packing of 6-bit scales and mins (same values as
// decode_scale, without a divergent branch).
struct ScaleBits {
    bool lo4;
    int xs_sc, xs_mn, ys;
    __device__ explicit ScaleBits(int l) {
        lo4 = l < 4;
        const int sh = 8 * (l & 3);
        xs_sc = sh;
        xs_mn = sh + (lo4 ? 0 : 4);
        ys = sh + (lo4 ? 4 : 6);
    }
};
__device__ __forceinline__ void decode_scale_bits(const ScaleBits &B, u32x4 h, float &ds,
                                                  float &dm) {
    const unsigned xsc = B.lo4 ? h.y : h.w, xmn = B.lo4 ? h.z : h.w;
    const unsigned sc = __builtin_amdgcn_ubfe(xsc, B.xs_sc, 4) |
                        (__builtin_amdgcn_ubfe(h.y, B.ys, 2) << 4);
    const unsigned mn = __builtin_amdgcn_ubfe(xmn, B.xs_mn, 4) |
                        (__builtin_amdgcn_ubfe(h.z, B.ys, 2) << 4);
    ds = half_lo(h.x) * (float)sc;
    dm = half_hi(h.x) * (float)mn;
}

// Low / high nibbles of the lane's 16-byte quant chunk, as 4 x 4 packed int8.
__device__ __forceinline__ void unpack_nibbles(u32x4 qw, int qlo[4], int qhi[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        qlo[k] = (int)(qw[k] & 0x0F0F0F0Fu);
        qhi[k] = (int)((qw[k] >> 4) & 0x0F0F0F0Fu);
    }
}

// sdot4 with a zero accumulator in one instruction (the three-operand form
// takes the constant; the builtin would first move 0 into a register).
__device__ __forceinline__ int sdot4_zero(int a, int b) {
    int r;
    asm("v_dot4_i32_i8 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Exact int32 dot of sub-block j = l: this lane's half plus its partner's half.
// cA pairs with the low nibbles, cB with the high nibbles.
__device__ __forceinline__ int subblock_dot(const LaneMap &L, const int qlo[4], const int qhi[4],
                                            i32x4 cA, i32x4 cB) {
    int dA = sdot4_zero(qlo[0], cA[0]), dB = sdot4_zero(qhi[0], cB[0]);
#pragma unroll
    for (int k = 1; k < 4; ++k) {
        dA = __builtin_amdgcn_sdot4(qlo[k], cA[k], dA, false);
        dB = __builtin_amdgcn_sdot4(qhi[k], cB[k], dB, false);
    }
    // lane h=0 keeps sub-block 2g (A halves), lane h=1 sub-block 2g+1 (B halves)
    const int keep = L.h ? dB : dA;
    const int send = L.h ? dA : dB;
    return keep + dpp_i<kQuadSwap1>(send);
}

}  // namespace q4k
