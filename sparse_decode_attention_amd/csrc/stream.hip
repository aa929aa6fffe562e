// Diagnostic: a plain streaming read of a device buffer, used to measure the
// practical HBM read bandwidth at the working-set sizes of decode (the
// ceiling the decode kernel's bandwidth is compared with). Not part of SparK.
#include "common.h"
#include "kernels.h"

namespace spark {

// Every thread reads 16-byte chunks with a grid stride, four in flight, and
// folds them with XOR; one word per block is written so nothing is elided.
__global__ void __launch_bounds__(256)
read_stream_kernel(const uint4* __restrict__ src, size_t n16, uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const uint4 a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    acc = (uint32_t)__reduce_xor_sync(0xffffffffffffffffull, (int)acc);
    if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const uint4*>(src), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace spark
