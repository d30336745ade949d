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

__device__ __forceinline__ u32x4 load_stream16(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
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

// Low / high nibbles of the lane's 16-byte quant chunk, as 4 x 4 packed int8.
__device__ __forceinline__ void unpack_nibbles(u32x4 qw, int qlo[4], int qhi[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        qlo[k] = (int)(qw[k] & 0x0F0F0F0Fu);
        qhi[k] = (int)((qw[k] >> 4) & 0x0F0F0F0Fu);
    }
}

// Exact int32 dot of sub-block j = l: this lane's half plus its partner's half.
// cA pairs with the low nibbles, cB with the high nibbles.
__device__ __forceinline__ int subblock_dot(const LaneMap &L, const int qlo[4], const int qhi[4],
                                            i32x4 cA, i32x4 cB) {
    int dA = 0, dB = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        dA = __builtin_amdgcn_sdot4(qlo[k], cA[k], dA, false);
        dB = __builtin_amdgcn_sdot4(qhi[k], cB[k], dB, false);
    }
    // lane h=0 keeps sub-block 2g (A halves), lane h=1 sub-block 2g+1 (B halves)
    const int keep = L.h ? dB : dA;
    const int send = L.h ? dA : dB;
    return keep + dpp_i<kQuadSwap1>(send);
}

}  // namespace q4k
