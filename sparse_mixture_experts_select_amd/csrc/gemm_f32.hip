// gemm_f32.hip -- the expert contractions in binary32 (fp32 storage and
// arithmetic), for small fp32 layers.
//
// Same per-expert products as the bf16 path (Mixtral of Experts, wikillm.com
// card, "Method", SwiGLU pseudocode): on the grouped rows of expert e,
//   h = SiLU(X_e . w1[e]) * (X_e . w3[e]),   y = h_e . w2[e].
// One thread per output element, contraction in ascending k with fp32 fused
// multiply-adds; a 64-column strip of one row per workgroup, so the weight
// reads of a workgroup are coalesced and the row of X or h is shared through
// the cache.  Meant for widths where the bf16 MFMA path does not apply.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ int expert_of_row(const int32_t* __restrict__ offsets, int E, int r) {
    int e = 0;
    while (e + 1 < E && offsets[e + 1] <= r) ++e;
    return e;
}

__global__ __launch_bounds__(64) void gemm1_swiglu_f32_kernel(
    const float* __restrict__ A, const float* __restrict__ W1, const float* __restrict__ W3,
    const int32_t* __restrict__ offsets, int R, int E, int K, int N, float* __restrict__ h) {
    const int col = blockIdx.x * 64 + threadIdx.x;
    for (int r = blockIdx.y; r < R; r += gridDim.y) {
        const int e = expert_of_row(offsets, E, r);
        if (col >= N) continue;
        const float* a = A + (size_t)r * K;
        const float* w1 = W1 + (size_t)e * K * N + col;
        const float* w3 = W3 + (size_t)e * K * N + col;
        float s1 = 0.0f, s3 = 0.0f;
        for (int kk = 0; kk < K; ++kk) {
            const float av = a[kk];
            s1 = fmaf(av, w1[(size_t)kk * N], s1);
            s3 = fmaf(av, w3[(size_t)kk * N], s3);
        }
        h[(size_t)r * N + col] = silu_f32(s1) * s3;
    }
}

__global__ __launch_bounds__(64) void gemm2_f32_kernel(const float* __restrict__ H,
                                                       const float* __restrict__ W2,
                                                       const int32_t* __restrict__ offsets, int R,
                                                       int E, int K, int N, float* __restrict__ y) {
    const int col = blockIdx.x * 64 + threadIdx.x;
    for (int r = blockIdx.y; r < R; r += gridDim.y) {
        const int e = expert_of_row(offsets, E, r);
        if (col >= N) continue;
        const float* hrow = H + (size_t)r * K;
        const float* w2 = W2 + (size_t)e * K * N + col;
        float s = 0.0f;
        for (int kk = 0; kk < K; ++kk) s = fmaf(hrow[kk], w2[(size_t)kk * N], s);
        y[(size_t)r * N + col] = s;
    }
}

dim3 grid_for(int R, int N) {
    int gy = R < 65535 ? R : 65535;
    if (gy < 1) gy = 1;
    return dim3((unsigned)((N + 63) / 64), (unsigned)gy);
}

}  // namespace

hipError_t launch_gemm1_swiglu_f32(const void* x_perm, const void* w1, const void* w3,
                                   const int32_t* offsets, int R, int E, int d, int f, void* h,
                                   hipStream_t stream) {
    hipLaunchKernelGGL(gemm1_swiglu_f32_kernel, grid_for(R, f), dim3(64), 0, stream,
                       reinterpret_cast<const float*>(x_perm), reinterpret_cast<const float*>(w1),
                       reinterpret_cast<const float*>(w3), offsets, R, E, d, f,
                       reinterpret_cast<float*>(h));
    return hipGetLastError();
}

hipError_t launch_gemm2_f32(const void* h, const void* w2, const int32_t* offsets, int R, int E,
                            int f, int d, float* y, hipStream_t stream) {
    hipLaunchKernelGGL(gemm2_f32_kernel, grid_for(R, d), dim3(64), 0, stream,
                       reinterpret_cast<const float*>(h), reinterpret_cast<const float*>(w2),
                       offsets, R, E, f, d, y);
    return hipGetLastError();
}

}  // namespace moe
