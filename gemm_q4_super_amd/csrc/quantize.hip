// Q8 activation quantizer (and the SwiGLU variant used by the routed-expert
// layer between its gate/up and down products).
//
// Per block of 32 fp32 values: amax = max|x|, scale = fl32(amax / 127), code =
// clamp(rne(fl32(x / scale)), -127, 127), sum = sum of codes; scale 0 gives
// codes 0.  quantize_block8 (q4k_device.h) computes every quotient correctly
// rounded, so codes are bit-exact with the definition.
//
// Mapping: 8 lanes per block, each lane owns 4 consecutive values (one 16-byte
// load); amax and sum reduce over the 8 lanes with DPP.  One wave covers 8
// blocks, a 256-thread workgroup 32 blocks.  HBM-bound and tiny next to the
// weight stream it feeds.
#include "q4k_device.h"
#include "q4k_internal.h"

namespace q4k {
namespace {

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
    if (GATED) v = swiglu4(*reinterpret_cast<const f32x4 *>(gate + off), v);
    const Q8Lane q = quantize_block8(v);
    *reinterpret_cast<unsigned *>(codes + off) = q.codes;
    if (sub == 0) {
        scales[blk] = q.d;
        sums[blk] = q.sum;
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
