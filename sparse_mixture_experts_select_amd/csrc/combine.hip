// combine.hip -- gate-weighted un-permute of the expert outputs, and RMSNorm.
//
// Mixtral of Experts (wikillm.com card, "Method"): the token's output is the
// sum over its k kept experts of gate * expert output, starting from zero
// (section 2.1 displays 1 and 3, moe_feed_forward pseudocode).  The expert
// outputs sit in grouped-row order; slot_row maps token t's j-th pick to its
// row.  Sums run in fp32 in a fixed order (K-split partials first, then picks
// j = 0..k-1), so results are bitwise reproducible.  With a residual the sum
// is residual + layer output, rounded once to the storage type.
//
// RMSNorm (unit gain) serves the stacked form h = h + MoE(RMSNorm(h)); the
// pages leave the normalisation to the code ("Method", steps for one token,
// item 5).  One workgroup per row, fp32 sum of squares, one rounding.  The
// router's fused form (router.hip) accumulates in exactly this order, so the
// two give the same bits.
#include "common.h"

namespace moe {
namespace {

constexpr int kPickBatch = 8;   // picks whose rows and gates are loaded together
constexpr int kMaxSlices = 16;  // K-slice partials of y (the host plans at most 16)

template <typename T> struct Io;
template <> struct Io<bf16> {
    __device__ static void load4(const void* p, size_t i, float* v) {
        const uint2 q = reinterpret_cast<const uint2*>(p)[i];
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
    }
    __device__ static void store4(void* p, size_t i, const float* v) {
        uint2 q;
        q.x = pack_bf16x2(v[0], v[1]);
        q.y = pack_bf16x2(v[2], v[3]);
        reinterpret_cast<uint2*>(p)[i] = q;
    }
};
template <> struct Io<float> {
    __device__ static void load4(const void* p, size_t i, float* v) {
        const float4 q = reinterpret_cast<const float4*>(p)[i];
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static void store4(void* p, size_t i, const float* v) {
        reinterpret_cast<float4*>(p)[i] = make_float4(v[0], v[1], v[2], v[3]);
    }
};

// 16-byte slices: 8 bf16 or 4 fp32 elements.
template <typename T> struct Io16;
template <> struct Io16<bf16> {
    static constexpr int N = 8;
    __device__ static void load(const void* p, size_t i, float* v) {
        const uint4 q = reinterpret_cast<const uint4*>(p)[i];
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ static void store(void* p, size_t i, const float* v) {
        reinterpret_cast<uint4*>(p)[i] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                                                    pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
    }
};
template <> struct Io16<float> {
    static constexpr int N = 4;
    __device__ static void load(const void* p, size_t i, float* v) { Io<float>::load4(p, i, v); }
    __device__ static void store(void* p, size_t i, const float* v) { Io<float>::store4(p, i, v); }
};

// One token per workgroup iteration; each thread takes 4 float4 columns
// (256 apart) of every pick at once, so all of a token's loads are in flight
// together.  Per column the sum order is fixed: picks j = 0..k-1 in slot
// order, g_j times the expert output added to the running sum (from zero).
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ gates,
                                                      const int32_t* __restrict__ slot_row,
                                                      const void* residual, int Tn, int d, int k,
                                                      void* out) {
    constexpr int U = 4;
    const int d4 = d / 4;
    for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
        for (int c0 = threadIdx.x; c0 < d4; c0 += 256 * U) {
            float4 acc[U];
#pragma unroll
            for (int u = 0; u < U; ++u) acc[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            // the residual is loaded up front, so its loads are in flight with
            // the expert outputs' (each element is read before this thread
            // writes it, so residual == out is fine)
            float rv[U][4];
            if (residual != nullptr) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + 256 * u;
                    if (c < d4) Io<T>::load4(residual, (size_t)t * d4 + c, rv[u]);
                }
            }
            // picks in batches of kPickBatch (one batch for k <= 8), in slot
            // order
            for (int j0 = 0; j0 < k; j0 += kPickBatch) {
                int rows[kPickBatch];
                float g[kPickBatch];
#pragma unroll
                for (int j = 0; j < kPickBatch; ++j) {
                    rows[j] = j0 + j < k ? slot_row[(size_t)t * k + j0 + j] : 0;
                    g[j] = j0 + j < k ? gates[(size_t)t * k + j0 + j] : 0.0f;
                }
#pragma unroll
                for (int j = 0; j < kPickBatch; ++j) {
                    if (j0 + j >= k) break;
                    const float4* yr = reinterpret_cast<const float4*>(y + (size_t)rows[j] * d);
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const int c = c0 + 256 * u;
                        const float4 sv = c < d4 ? yr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
                        acc[u].x += g[j] * sv.x; acc[u].y += g[j] * sv.y;
                        acc[u].z += g[j] * sv.z; acc[u].w += g[j] * sv.w;
                    }
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = c0 + 256 * u;
                if (c >= d4) continue;
                const size_t idx = (size_t)t * d4 + c;
                float a[4] = {acc[u].x, acc[u].y, acc[u].z, acc[u].w};
                if (residual != nullptr)
                    for (int q = 0; q < 4; ++q) a[q] = rv[u][q] + a[q];
                Io<T>::store4(out, idx, a);
            }
        }
    }
}

// The same with y in `splits` K-slice partials (the streamed path's GEMM 2
// cuts K across workgroups).  One thread per (token, float4 column), columns
// over blockIdx.x and tokens over blockIdx.y, so a batch of a few tokens
// still spreads over many workgroups; all of a pick's slices are loaded at
// once, then added in slice order before g_j times their sum is added.
template <typename T>
__global__ __launch_bounds__(256) void combine_slices_kernel(const float* __restrict__ y, int splits,
                                                             size_t split_stride,
                                                             const float* __restrict__ gates,
                                                             const int32_t* __restrict__ slot_row,
                                                             const void* residual, int Tn, int d,
                                                             int k, void* out) {
    const int d4 = d / 4;
    const int c = blockIdx.x * 256 + threadIdx.x;
    if (c >= d4) return;
    const size_t stride4 = split_stride / 4;
    for (int t = blockIdx.y; t < Tn; t += gridDim.y) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const float4* yr = reinterpret_cast<const float4*>(y + (size_t)slot_row[(size_t)t * k + j] * d) + c;
            const float gj = gates[(size_t)t * k + j];
            float4 v[kMaxSlices];
#pragma unroll
            for (int p = 0; p < kMaxSlices; ++p)
                if (p < splits) v[p] = yr[p * stride4];
            float4 sv = v[0];
#pragma unroll
            for (int p = 1; p < kMaxSlices; ++p) {
                if (p < splits) {
                    sv.x += v[p].x; sv.y += v[p].y; sv.z += v[p].z; sv.w += v[p].w;
                }
            }
            acc.x += gj * sv.x; acc.y += gj * sv.y; acc.z += gj * sv.z; acc.w += gj * sv.w;
        }
        const size_t idx = (size_t)t * d4 + c;
        float a[4] = {acc.x, acc.y, acc.z, acc.w};
        if (residual != nullptr) {
            float rv[4];
            Io<T>::load4(residual, idx, rv);
            for (int q = 0; q < 4; ++q) a[q] = rv[q] + a[q];
        }
        Io<T>::store4(out, idx, a);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const void* h, void* x, int Tn, int d,
                                                      float eps) {
    __shared__ float part[4];
    constexpr int N = Io16<T>::N;
    const int ds = d / N;  // 16-byte slices per row
    for (int t = blockIdx.x; t < Tn; t += gridDim.x) {
        float ss = 0.0f;
        for (int c = threadIdx.x; c < ds; c += 256) {
            float v[N];
            Io16<T>::load(h, (size_t)t * ds + c, v);
#pragma unroll
            for (int u = 0; u < N; ++u) ss = fmaf(v[u], v[u], ss);
        }
        for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
        if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
        __syncthreads();
        const float r = 1.0f / sqrtf((part[0] + part[1] + part[2] + part[3]) / (float)d + eps);
        for (int c = threadIdx.x; c < ds; c += 256) {
            float v[N];
            Io16<T>::load(h, (size_t)t * ds + c, v);
#pragma unroll
            for (int u = 0; u < N; ++u) v[u] *= r;
            Io16<T>::store(x, (size_t)t * ds + c, v);
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_combine(int dtype, const float* y, int splits, const float* gates,
                          const int32_t* slot_row, const void* residual, int T, int d, int k, int R,
                          void* out, hipStream_t stream) {
    if (splits < 1 || splits > kMaxSlices) return hipErrorInvalidValue;
    if (splits > 1) {
        const dim3 grid((unsigned)((d / 4 + 255) / 256), (unsigned)(T < 65535 ? (T > 0 ? T : 1) : 65535));
        const size_t split_stride = (size_t)R * d;
        if (dtype == 0)
            hipLaunchKernelGGL(combine_slices_kernel<bf16>, grid, dim3(256), 0, stream, y, splits,
                               split_stride, gates, slot_row, residual, T, d, k, out);
        else
            hipLaunchKernelGGL(combine_slices_kernel<float>, grid, dim3(256), 0, stream, y, splits,
                               split_stride, gates, slot_row, residual, T, d, k, out);
        return hipGetLastError();
    }
    int blocks = T < 16384 ? T : 16384;
    if (blocks < 1) blocks = 1;
    if (dtype == 0)
        hipLaunchKernelGGL(combine_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, y, gates,
                           slot_row, residual, T, d, k, out);
    else
        hipLaunchKernelGGL(combine_kernel<float>, dim3(blocks), dim3(256), 0, stream, y, gates,
                           slot_row, residual, T, d, k, out);
    return hipGetLastError();
}

hipError_t launch_rmsnorm(int dtype, const void* h, void* x, int T, int d, float eps,
                          hipStream_t stream) {
    int blocks = T < 16384 ? T : 16384;
    if (blocks < 1) blocks = 1;
    if (dtype == 0)
        hipLaunchKernelGGL(rmsnorm_kernel<bf16>, dim3(blocks), dim3(256), 0, stream, h, x, T, d, eps);
    else
        hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(blocks), dim3(256), 0, stream, h, x, T, d,
                           eps);
    return hipGetLastError();
}

}  // namespace moe
