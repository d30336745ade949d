// Measurement aids: the practical ceilings the decode launches are compared
// with -- a plain 16-byte stream read over a buffer (the bytes a GEMV launch
// must move, with no arithmetic) and an empty kernel (the cost of a kernel
// boundary alone) -- and, for the prefill GEMM, whether fp16 matrix-core ops
// and fp32 vector fmas issued by two waves of one SIMD run concurrently.
// None is on the product path.
#include "q4k_internal.h"

namespace q4k {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Every thread reads 16-byte chunks in a grid-stride loop and folds them with
// xor; one word per workgroup is written so the loads are not dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ src,
                                                          int64_t chunks, unsigned *__restrict__ sink) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < chunks; i += stride) acc ^= src[i];
    unsigned v = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v ^= __shfl_xor(v, o);
    __shared__ unsigned part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

__global__ void empty_kernel() {}

// 8 waves: waves 0-3 (one per SIMD) run `iters` rounds of four independent
// v_mfma_f32_32x32x16_f16 chains when bit 0 of `what` is set; waves 4-7 (one
// per SIMD, beside them) run `iters * vrep` rounds of 32 fp32 fmas in sixteen
// independent chains when bit 1 is set.  The sums of both are folded into one
// word per workgroup.
__global__ __launch_bounds__(512) void mfma_valu_kernel(int64_t iters, int vrep, int what,
                                                        float *__restrict__ sink) {
    const int w = threadIdx.x >> 6;
    float s = 0.0f;
    if (w >= 4) {
        if (what & 2) {
            float a[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) a[k] = (float)threadIdx.x * 0.001f + (float)k;
            const int64_t n = iters * vrep;
#pragma unroll 1
            for (int64_t it = 0; it < n; ++it)
#pragma unroll
                for (int r = 0; r < 2; ++r)
#pragma unroll
                    for (int k = 0; k < 16; ++k) a[k] = fmaf(a[k], 0.999f, 0.001f);
#pragma unroll
            for (int k = 0; k < 16; ++k) s += a[k];
        }
    } else if (what & 1) {
        const _Float16 one = (_Float16)((threadIdx.x & 7) == 0 ? 1.0f : 0.0f);
        const half8 A = {one, one, one, one, one, one, one, one};
        f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
#pragma unroll 1
        for (int64_t it = 0; it < iters; ++it) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, A, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, A, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, A, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(A, A, c3, 0, 0, 0);
        }
        s = c0[0] + c1[1] + c2[2] + c3[3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    __shared__ float part[8];
    if ((threadIdx.x & 63) == 0) part[w] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k) t += part[k];
        sink[blockIdx.x] = t;
    }
}

}  // namespace

hipError_t launch_stream_read(const void *buf, int64_t bytes, int64_t grid, unsigned *sink,
                              hipStream_t stream) {
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

hipError_t launch_empty(int64_t grid, hipStream_t stream) {
    hipLaunchKernelGGL(empty_kernel, dim3((unsigned)grid), dim3(64), 0, stream);
    return hipGetLastError();
}

hipError_t launch_mfma_valu(int64_t grid, int64_t iters, int vrep, int what, float *sink,
                            hipStream_t stream) {
    hipLaunchKernelGGL(mfma_valu_kernel, dim3((unsigned)grid), dim3(512), 0, stream, iters, vrep,
                       what, sink);
    return hipGetLastError();
}

}  // namespace q4k
