// Measurement aids: the practical ceilings the decode launches are compared
// with.  A plain 16-byte stream read over a buffer (the bytes a GEMV launch
// must move, with no arithmetic) and an empty kernel (the cost of a kernel
// boundary alone).  Neither is on the product path.
#include "q4k_internal.h"

namespace q4k {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

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

}  // namespace q4k
