// Diagnostic: a plain streaming read of a device buffer, used to measure the
// practical HBM read bandwidth at the working-set sizes of decode (the
// ceiling the decode kernel's bandwidth is compared with). Not part of SparK.
#include "common.h"
#include "kernels.h"

namespace spark {

// Every thread reads 16-byte chunks with a grid stride, four in flight, and
// folds them with XOR; one word per block is written so nothing is elided.
// The requests are nontemporal, as decode's V requests are (each wave's
// request covers whole lines that are never read again).
typedef uint32_t u32x4_nt __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t fold(const u32x4_nt* p) {
    const u32x4_nt x = __builtin_nontemporal_load(p);
    return x.x ^ x.y ^ x.z ^ x.w;
}
__global__ void __launch_bounds__(256)
read_stream_kernel(const u32x4_nt* __restrict__ src, size_t n16, uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride)
        acc ^= fold(src + i) ^ fold(src + i + stride) ^ fold(src + i + 2 * stride) ^ fold(src + i + 3 * stride);
    for (; i < n16; i += stride) acc ^= fold(src + i);
    acc = (uint32_t)__reduce_xor_sync(0xffffffffffffffffull, (int)acc);
    if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

hipError_t launch_read_stream(const void* src, size_t bytes, uint32_t* sink, int blocks, hipStream_t stream) {
    hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(256), 0, stream,
                       static_cast<const u32x4_nt*>(src), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace spark
