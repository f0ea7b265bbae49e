// router.hip -- router logits, top-k select and softmax over the kept logits.
//
// Mixtral of Experts (wikillm.com card, "Method"): a bias-free linear router
// gives one logit per expert (section 2.1, steps-for-one-token item 2); the K
// largest are kept and a softmax is taken over those K only, so their weights
// sum to one (section 2.1 display 2; "Pitfalls": renormalised top-2 weights,
// softmax in fp32).
//
// One wavefront handles TPW tokens at a time.  The router matrix [d,E] is
// staged once per workgroup in LDS when it fits (64 KiB for d=4096, E=8 in
// bf16), transposed to [E][d] so that a lane reads the 16 contiguous bytes of
// one expert's column that match its 16-byte slice of x (consecutive lanes,
// consecutive addresses: no bank conflicts).  Each lane accumulates fp32
// partial logits over a strided set of 16-byte slices of d, a butterfly of
// cross-lane adds gives every lane the full logits, and the selection runs
// redundantly on all lanes; lane 0 stores it.
//
// Logits stay fp32 (products of bf16 inputs are exact in fp32, sums are
// fp32).  Ties break toward the lower expert index; the picks are stored by
// descending logit.  An optional fp32 bias [E] is added before selection.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxK = 8;
constexpr int kLdsBytes = 64 * 1024;

template <typename T> struct Vec;
template <> struct Vec<bf16> {
    static constexpr int N = 8;  // elements per 16-byte load
    __device__ static void load(const bf16* p, float* v) {
        uint4 q = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ static float one(const bf16* p, int i) { return (float)p[i]; }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    __device__ static void load(const float* p, float* v) {
        float4 q = *reinterpret_cast<const float4*>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static float one(const float* p, int i) { return p[i]; }
};

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

template <typename T, int EMAX, int TPW>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ bias, int T_,
    int d, int E, int k, int use_lds, int32_t* __restrict__ ids, float* __restrict__ gates) {
    extern __shared__ __align__(16) unsigned char lds_raw[];
    T* wt = reinterpret_cast<T*>(lds_raw);  // [E][d] when use_lds
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    constexpr int VN = Vec<T>::N;

    if (use_lds) {
        // Transposing copy: flat element q of w_router is (i, e) = (q / E, q % E);
        // (i, e) advance incrementally, so the loop has no division.
        const int n = d * E;
        const int step = kThreads * VN;
        const int di = step / E, de = step - (step / E) * E;
        int q0 = threadIdx.x * VN;
        int i0 = q0 / E, e0 = q0 - i0 * E;
        for (; q0 < n; q0 += step) {
            float v[VN];
            Vec<T>::load(wr + q0, v);
            int i = i0, e = e0;
#pragma unroll
            for (int u = 0; u < VN; ++u) {
                wt[(size_t)e * d + i] = (T)v[u];
                if (++e == E) {
                    e = 0;
                    ++i;
                }
            }
            i0 += di;
            e0 += de;
            if (e0 >= E) {
                e0 -= E;
                ++i0;
            }
        }
        __syncthreads();
    }

    const int stride = 64 * VN;
    const int groups = (T_ + TPW - 1) / TPW;
    for (int grp = blockIdx.x * kWaves + wave; grp < groups; grp += gridDim.x * kWaves) {
        const int t0 = grp * TPW;
        float acc[TPW][EMAX];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int e = 0; e < EMAX; ++e) acc[tt][e] = 0.0f;

        for (int i0 = lane * VN; i0 < d; i0 += stride) {
            float xv[TPW][VN];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                if (t0 + tt < T_) {
                    Vec<T>::load(x + (size_t)(t0 + tt) * d + i0, xv[tt]);
                } else {
#pragma unroll
                    for (int u = 0; u < VN; ++u) xv[tt][u] = 0.0f;
                }
            }
#pragma unroll
            for (int e = 0; e < EMAX; ++e) {
                if (e < E) {
                    float w[VN];
                    if (use_lds) {
                        Vec<T>::load(wt + (size_t)e * d + i0, w);
                    } else {
#pragma unroll
                        for (int u = 0; u < VN; ++u) w[u] = Vec<T>::one(wr, (i0 + u) * E + e);
                    }
#pragma unroll
                    for (int u = 0; u < VN; ++u)
#pragma unroll
                        for (int tt = 0; tt < TPW; ++tt) acc[tt][e] = fmaf(xv[tt][u], w[u], acc[tt][e]);
                }
            }
        }

#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            const int t = t0 + tt;
            float l[EMAX];
#pragma unroll
            for (int e = 0; e < EMAX; ++e) {
                l[e] = (e < E) ? wave_sum(acc[tt][e]) : 0.0f;
                if (bias != nullptr && e < E) l[e] += bias[e];
            }
            if (t >= T_) continue;
            // k rounds of argmax over the experts not yet taken; strict '>'
            // in ascending expert order keeps the lowest index on ties.
            uint64_t taken = 0;
            int sel[kMaxK];
            float sv[kMaxK];
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k) {
                    int best = -1;
                    float bv = 0.0f;
#pragma unroll
                    for (int e = 0; e < EMAX; ++e) {
                        const bool free_e = (e < E) && !((taken >> e) & 1ull);
                        if (free_e && (best < 0 || l[e] > bv)) {
                            best = e;
                            bv = l[e];
                        }
                    }
                    taken |= 1ull << best;
                    sel[j] = best;
                    sv[j] = bv;
                }
            }
            // softmax over the k kept logits; sv[0] is the largest.
            float p[kMaxK];
            float z = 0.0f;
#pragma unroll
            for (int j = 0; j < kMaxK; ++j) {
                if (j < k) {
                    p[j] = expf(sv[j] - sv[0]);
                    z += p[j];
                }
            }
            const float rz = 1.0f / z;
            if (lane == 0) {
#pragma unroll
                for (int j = 0; j < kMaxK; ++j) {
                    if (j < k) {
                        ids[(size_t)t * k + j] = sel[j];
                        gates[(size_t)t * k + j] = p[j] * rz;
                    }
                }
            }
        }
    }
}

template <typename T, int EMAX, int TPW>
hipError_t launch_t(const void* x, const void* wr, const float* bias, int T_, int d, int E, int k,
                    int32_t* ids, float* gates, hipStream_t stream) {
    const size_t wbytes = (size_t)d * E * sizeof(T);
    const int use_lds = wbytes <= (size_t)kLdsBytes ? 1 : 0;
    const int groups = (T_ + TPW - 1) / TPW;
    int blocks = (groups + kWaves - 1) / kWaves;
    // Enough workgroups to cover every CU a few times; each stages the
    // router matrix once and then loops over its share of tokens.
    const int max_blocks = 1024;
    if (blocks > max_blocks) blocks = max_blocks;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL((router_topk_kernel<T, EMAX, TPW>), dim3(blocks), dim3(kThreads),
                       use_lds ? wbytes : 0, stream, reinterpret_cast<const T*>(x),
                       reinterpret_cast<const T*>(wr), bias, T_, d, E, k, use_lds, ids, gates);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_e(const void* x, const void* wr, const float* bias, int T_, int d, int E,
                      int k, int32_t* ids, float* gates, hipStream_t stream) {
    // Small batches: one token per wave, to spread them over more CUs.
    if (E <= 8 && T_ <= 2048) return launch_t<T, 8, 1>(x, wr, bias, T_, d, E, k, ids, gates, stream);
    if (E <= 8) return launch_t<T, 8, 4>(x, wr, bias, T_, d, E, k, ids, gates, stream);
    if (E <= 16) return launch_t<T, 16, 2>(x, wr, bias, T_, d, E, k, ids, gates, stream);
    if (E <= 32) return launch_t<T, 32, 1>(x, wr, bias, T_, d, E, k, ids, gates, stream);
    return launch_t<T, 64, 1>(x, wr, bias, T_, d, E, k, ids, gates, stream);
}

}  // namespace

hipError_t launch_router_topk(int dtype, const void* x, const void* w_router, const float* bias,
                              int T, int d, int E, int k, int32_t* ids, float* gates,
                              hipStream_t stream) {
    if (dtype == 0) return dispatch_e<bf16>(x, w_router, bias, T, d, E, k, ids, gates, stream);
    return dispatch_e<float>(x, w_router, bias, T, d, E, k, ids, gates, stream);
}

}  // namespace moe
