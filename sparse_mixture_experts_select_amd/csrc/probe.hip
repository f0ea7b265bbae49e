// probe.hip -- a plain streaming read of a device buffer, the measured
// ceiling that the weight-streaming (HBM-bound) kernels are compared with
// beside the 8 TB/s datasheet figure.  Not part of the layer.
//
// Each thread reads 16-byte vectors in a grid-stride loop, four in flight per
// iteration, and folds them with XOR so no load is dead; one atomic per wave
// writes the fold to `sink` (its value has no meaning).
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t fold(const uint4& v) { return v.x ^ v.y ^ v.z ^ v.w; }

__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
        acc ^= fold(a) ^ fold(b) ^ fold(c) ^ fold(d);
    }
    for (; i < n16; i += stride) acc ^= fold(p[i]);
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, int blocks, uint32_t* sink,
                             hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace moe
