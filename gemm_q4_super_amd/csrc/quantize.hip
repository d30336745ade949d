// Q8 activation quantizer (and the SwiGLU variant used by the routed-expert
// layer between its gate/up and down products).
//
// Per block of 32 fp32 values: amax = max|x|, scale = fl32(amax / 127), code =
// clamp(rne(fl32(x / scale)), -127, 127), sum = sum of codes; scale 0 gives
// codes 0.  Division and rounding are IEEE fp32 (hipcc's default correctly
// rounded division, v_rndne_f32), so codes are bit-exact with the definition.
//
// Mapping: 8 lanes per block, each lane owns 4 consecutive values (one 16-byte
// load); amax and sum reduce over the 8 lanes with DPP.  One wave covers 8
// blocks, a 256-thread workgroup 32 blocks.  HBM-bound and tiny next to the
// weight stream it feeds.
#include "q4k_internal.h"

namespace q4k {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// DPP helpers: reductions over aligned groups of 8 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141; // lane i <-> 7-i within each 8 lanes

__device__ __forceinline__ float group8_max(float v) {
    v = fmaxf(v, dpp_f<kQuadSwap1>(v));
    v = fmaxf(v, dpp_f<kQuadSwap2>(v));
    v = fmaxf(v, dpp_f<kRowHalfMirror>(v));
    return v;
}
__device__ __forceinline__ int group8_sum(int v) {
    v += dpp_i<kQuadSwap1>(v);
    v += dpp_i<kQuadSwap2>(v);
    v += dpp_i<kRowHalfMirror>(v);
    return v;
}

__device__ __forceinline__ int quant1(float x, float d) {
    if (d == 0.0f) return 0;
    float r = __builtin_rintf(x / d);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

template <bool GATED>
__global__ __launch_bounds__(256) void quantize_kernel(const float *__restrict__ x,
                                                       const float *__restrict__ gate,
                                                       int64_t nblocks,
                                                       int8_t *__restrict__ codes,
                                                       float *__restrict__ scales,
                                                       int32_t *__restrict__ sums) {
    const int64_t blk = (int64_t)blockIdx.x * 32 + (threadIdx.x >> 3);
    const int sub = threadIdx.x & 7;
    // Every lane of a block's 8-lane group takes the same branch, so the DPP
    // reductions below only ever mix lanes of live blocks.
    if (blk >= nblocks) return;
    const int64_t off = blk * 32 + sub * 4;
    f32x4 v = *reinterpret_cast<const f32x4 *>(x + off);
    if (GATED) {
        f32x4 g = *reinterpret_cast<const f32x4 *>(gate + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            double gd = (double)g[i];
            v[i] = (float)(gd / (1.0 + exp(-gd)) * (double)v[i]);
        }
    }
    float amax = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    amax = group8_max(amax);
    const float d = amax / 127.0f;
    int c0 = quant1(v[0], d), c1 = quant1(v[1], d), c2 = quant1(v[2], d), c3 = quant1(v[3], d);
    int packed = (c0 & 0xFF) | ((c1 & 0xFF) << 8) | ((c2 & 0xFF) << 16) | ((int)((unsigned)c3 << 24));
    *reinterpret_cast<int *>(codes + off) = packed;
    int s = group8_sum(c0 + c1 + c2 + c3);
    if (sub == 0) {
        scales[blk] = d;
        sums[blk] = s;
    }
}

}  // namespace

hipError_t launch_quantize(const float *x, int64_t M, int64_t K, const float *gate,
                           int8_t *codes, float *scales, int32_t *sums,
                           hipStream_t stream) {
    const int64_t nblocks = M * (K / kQB);
    const int64_t grid = (nblocks + 31) / 32;
    if (gate)
        hipLaunchKernelGGL(quantize_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream,
                           x, gate, nblocks, codes, scales, sums);
    else
        hipLaunchKernelGGL(quantize_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream,
                           x, gate, nblocks, codes, scales, sums);
    return hipGetLastError();
}

}  // namespace q4k
