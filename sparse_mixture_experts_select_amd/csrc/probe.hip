// probe.hip -- measurement aids, not part of the layer:
//
// read_probe_kernel: a streaming read of a device buffer, the measured
// ceiling that the weight-streaming (HBM-bound) kernels are compared with
// beside the 8 TB/s datasheet figure.  Each thread reads 16-byte vectors in a
// grid-stride loop, eight in flight per iteration, marked nontemporal (as the
// streamed GEMMs' weight loads are: HBM serves such a stream at ~7.2 TB/s,
// plain loads at ~6.4), and folds them with XOR so no load is dead; one
// atomic per wave writes the fold to `sink` (its value has no meaning).
//
// mfma_probe_kernel: bf16 matrix-core work with no memory traffic, the
// measured ceiling that the MFMA-bound tile GEMMs are compared with beside
// the 2.5 PFLOP/s datasheet figure (which assumes 2.4 GHz; under a dense
// MFMA stream on random data the part holds a lower clock).  Each of the
// four waves of a workgroup runs the tile GEMMs' per-wave shape -- 8 x 8
// fragments of v_mfma_f32_16x16x32_bf16, 256 fp32 accumulators -- on 8 A and
// 8 B operand fragments read once from `ops` (random data, so operand bits
// toggle from one MFMA to the next as in a real product), paired differently
// in the two halves of an iteration; a 96 KiB LDS reservation keeps one
// workgroup per CU, as in the tile GEMMs.  Optionally records each workgroup's shader-clock cycles and
// 100 MHz real-time ticks, which give the clock held under that load.
#include "common.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t fold(const u32x4& v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 7 * stride < n16; i += 8 * stride) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc ^= fold(v[u]);
    }
    for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(p + i));
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

constexpr int kProbeHold = 24 * 1024;  // uint32 words of LDS reserved per workgroup

__global__ __launch_bounds__(256, 1) void mfma_probe_kernel(const uint4* __restrict__ ops, size_t n16,
                                                            int iters, uint32_t* __restrict__ sink,
                                                            unsigned long long* __restrict__ clocks) {
    __shared__ uint32_t hold[kProbeHold];
    // 16 consecutive 16-byte vectors per thread, wrapping at the end of ops
    // (n16 >= 1024)
    const size_t base = ((size_t)blockIdx.x * 256 + threadIdx.x) * 16 % n16;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const size_t j = base + i < n16 ? base + i : base + i - n16;
        const bf16x8 v = __builtin_bit_cast(bf16x8, ops[j]);
        if (i < 8) a[i] = v;
        else b[i - 8] = v;
    }
    floatx4 acc[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};
    hold[threadIdx.x] = 0u;
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    const unsigned long long t0 = __builtin_amdgcn_s_memrealtime();
    // Each MFMA accumulates in place in its AGPRs.  (Written as inline asm:
    // with loop-invariant operands the compiler otherwise rotates the
    // accumulators through other registers every iteration, which is not
    // the tile GEMMs' instruction stream.)
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int n = 0; n < 8; ++n)
#pragma unroll
                for (int m = 0; m < 8; ++m)
                    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0"
                                 : "+a"(acc[m][n])
                                 : "v"(a[(m + h) & 7]), "v"(b[(n + 3 * h) & 7]));
    }
    // let the last MFMAs retire before their accumulators are read
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    const unsigned long long t1 = __builtin_amdgcn_s_memrealtime();
    // (thread index formed afresh, so nothing lane-dependent is kept across
    // the loop beside the accumulators and operands)
    const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int tid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) * 64 + lane;
    uint32_t f = hold[tid];  // 0: only keeps the LDS reservation
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n)
            f ^= __float_as_uint(acc[m][n][0] + acc[m][n][1] + acc[m][n][2] + acc[m][n][3]);
    for (int off = 32; off >= 1; off >>= 1) f ^= __shfl_xor(f, off, 64);
    if (lane == 0) atomicXor(sink, f);
    if (clocks != nullptr && tid == 0) {
        clocks[2 * blockIdx.x] = c1 - c0;
        clocks[2 * blockIdx.x + 1] = t1 - t0;
    }
}

}  // namespace

hipError_t launch_mfma_probe(const void* ops, size_t bytes, int iters, int blocks, uint32_t* sink,
                             unsigned long long* clocks, hipStream_t stream) {
    hipLaunchKernelGGL(mfma_probe_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(ops), bytes / 16, iters, sink, clocks);
    return hipGetLastError();
}

hipError_t launch_read_probe(const void* buf, size_t bytes, int blocks, uint32_t* sink,
                             hipStream_t stream) {
    hipLaunchKernelGGL(read_probe_kernel, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace moe
