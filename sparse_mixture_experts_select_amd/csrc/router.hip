// router.hip -- router logits, top-k select and softmax over the kept logits.
//
// Mixtral of Experts (wikillm.com card, "Method"): a bias-free linear router
// gives one logit per expert (section 2.1, steps-for-one-token item 2); the K
// largest are kept and a softmax is taken over those K only, so their weights
// sum to one (section 2.1 display 2; "Pitfalls": renormalised top-2 weights,
// softmax in fp32).
//
// A workgroup of 4 wavefronts handles TPW consecutive tokens.  The hidden
// dimension is cut into 16-byte slices of x; lane l of wave w takes slices
// w*64 + l, w*64 + l + 256, ..., so every x load of a wave is one contiguous
// 1 KiB run.  For bf16 with E = 8 the matching router rows (8 rows of 8
// experts, 128 contiguous bytes) are read straight from global memory, where
// the 64 KiB router matrix stays L2-resident; other shapes read it element by
// element.  The TPW x E partial logits of a lane are summed across the lanes
// of a wave with a halving butterfly (each exchange step sends half as many
// values as the one before), then across the 4 waves in LDS in a fixed
// order; then one lane of wave 0 per (token, expert) finds that expert's
// rank among the token's logits, and the lanes of ranks 0..k-1 write the
// picks and their softmax weights (any k <= E <= 64).
//
// Logits stay fp32 (products of bf16 inputs are exact in fp32, sums are
// fp32).  Ties break toward the lower expert index; the picks are stored by
// descending logit.  An optional fp32 bias [E] is added before selection.
//
// Fused RMSNorm (NORM): the input rows are the residual stream h of the
// stacked block h = h + MoE(RMSNorm(h)).  A first pass over the row forms
// its sum of squares (keeping the slices in registers), the second scales each 16-byte slice by
// 1/sqrt(mean + eps), rounds it once to the storage type, stores it as the
// layer input x, and takes the logits from those rounded values.  The sum of
// squares is accumulated in the same order as rmsnorm_kernel (the same
// slices per thread, fmaf in element order, a butterfly over the wave, the
// four waves in order), so both forms give x bit for bit.
#include "common.h"

#include <atomic>

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
// Fused RMSNorm: the first kNormCache 16-byte slices of each of a lane's rows
// stay in registers between the two passes (all of a row up to d = 4096 in
// bf16), so the second pass reloads only what lies past them.
constexpr int kNormCache = 2;

template <typename T> struct Vec;
template <> struct Vec<bf16> {
    static constexpr int N = 8;  // elements per 16-byte load
    __device__ static void unpack(const uint4& q, float* v) {
        v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
        v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
    }
    __device__ static void load(const bf16* p, float* v) { unpack(*reinterpret_cast<const uint4*>(p), v); }
    __device__ static float one(const bf16* p, size_t i) { return (float)p[i]; }
    // The 8 values of q scaled by r, rounded, stored to p; q <- the stored words.
    __device__ static void scale_store_words(uint4& q, float* v, float r, bf16* p) {
        unpack(q, v);
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = pack_bf16x2(v[2 * i] * r, v[2 * i + 1] * r);
        q = make_uint4(w[0], w[1], w[2], w[3]);
        *reinterpret_cast<uint4*>(p) = q;
    }
    // v <- round(v * r), stored to p; v keeps the rounded values.
    __device__ static void scale_store(float* v, float r, bf16* p) {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            w[q] = pack_bf16x2(v[2 * q] * r, v[2 * q + 1] * r);
            v[2 * q] = bf16_lo(w[q]);
            v[2 * q + 1] = bf16_hi(w[q]);
        }
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};
template <> struct Vec<float> {
    static constexpr int N = 4;
    __device__ static void unpack(const uint4& q, float* v) {
        v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    }
    __device__ static void load(const float* p, float* v) { unpack(*reinterpret_cast<const uint4*>(p), v); }
    __device__ static float one(const float* p, size_t i) { return p[i]; }
    __device__ static void scale_store(float* v, float r, float* p) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] *= r;
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
};

template <int NV>
constexpr int log2_of() { return NV <= 1 ? 0 : 1 + log2_of<NV / 2>(); }

// Sum each of NV = 2^m per-lane values over the 64 lanes of a wave.  At
// offset o (32, 16, ...) the lane with bit o set keeps the upper half of its
// remaining values and sends the lower half to its partner, which does the
// reverse, so each step exchanges half as many values as the one before
// (NV - 1 shuffles in all, then 6 - m single ones).  On return v[0] of lane L
// holds the sum of value index (L >> (6 - m)) & (NV - 1).
template <int NV, int S>
__device__ __forceinline__ void wave_sum_step(float (&v)[NV], int lane) {
    constexpr int off = 32 >> S;
    constexpr int count = S < log2_of<NV>() ? (NV >> S) : 1;  // values still held
    if constexpr (count > 1) {
        constexpr int half = count / 2;
        const bool upper = (lane & off) != 0;
#pragma unroll
        for (int j = 0; j < half; ++j) {
            const float send = upper ? v[j] : v[j + half];
            const float keep = upper ? v[j + half] : v[j];
            v[j] = keep + __shfl_xor(send, off, 64);
        }
    } else {
        v[0] += __shfl_xor(v[0], off, 64);
    }
    if constexpr (S < 5) wave_sum_step<NV, S + 1>(v, lane);
}

template <int NV>
__device__ __forceinline__ void wave_sum_split(float (&v)[NV], int lane) {
    static_assert(NV >= 1 && NV <= 64 && (NV & (NV - 1)) == 0, "NV must be a power of 2 up to 64");
    wave_sum_step<NV, 0>(v, lane);
}

// LDS of the logit reduction and selection for TPW tokens.
template <int TPW, int EMAX>
struct RouterLds {
    float part[kWaves][TPW][EMAX];
    float logit[TPW][EMAX];
    float pexp[TPW][EMAX];
};

// The TPW x EMAX partial logits of every lane of the workgroup (acc[tt][e]
// stays 0 for e >= E) summed over a wave by the halving butterfly, then over
// the 4 waves in order; then the selection and softmax of tokens t0 ..
// t0 + TPW - 1.  Every thread of the workgroup must call it (it holds
// barriers); back-to-back calls need no barrier between them.
template <int TPW, int EMAX>
__device__ __forceinline__ void reduce_select(const float (&acc)[TPW][EMAX], RouterLds<TPW, EMAX>& sm,
                                              const float* __restrict__ bias, int t0, int T_, int E,
                                              int k, int32_t* __restrict__ ids,
                                              float* __restrict__ gates, int lane, int wave) {
    // value index tt * EMAX + e
    constexpr int NV = TPW * EMAX;
    constexpr int SHIFT = 6 - log2_of<NV>();
    float v[NV];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) v[tt * EMAX + e] = acc[tt][e];
    wave_sum_split<NV>(v, lane);
    if ((lane & ((1 << SHIFT) - 1)) == 0) (&sm.part[wave][0][0])[lane >> SHIFT] = v[0];
    __syncthreads();
    // Selection: lane (tt, e) of wave 0 holds token tt's logit of expert e
    // (TPW * EMAX <= 64 lanes).  Its stable rank -- the number of experts
    // before it in the order (logit descending, index ascending) -- is its
    // slot: rank j is what the j-th round of an argmax with strict '>' over
    // ascending indices would pick, so the k picks are the ranks 0..k-1 with
    // ties kept by the lower index, for any k <= E.
    static_assert(TPW * EMAX <= 64, "one lane of wave 0 per (token, expert)");
    const int tt = lane / EMAX;
    const int e = lane % EMAX;
    const int t = t0 + tt;
    const bool mine = wave == 0 && lane < TPW * EMAX && e < E && t < T_;
    float l = 0.0f;
    if (mine) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) l += sm.part[w][tt][e];
        if (bias != nullptr) l += bias[e];
        sm.logit[tt][e] = l;
    }
    __syncthreads();
    int rank = E;
    float p = 0.0f;
    if (mine) {
        rank = 0;
        float lmax = sm.logit[tt][0];
        for (int o = 0; o < E; ++o) {
            const float lo = sm.logit[tt][o];
            rank += (lo > l || (lo == l && o < e)) ? 1 : 0;
            lmax = fmaxf(lmax, lo);
        }
        // softmax over the k kept logits, max-subtracted (the rank-0 logit)
        if (rank < k) {
            p = expf(l - lmax);
            sm.pexp[tt][rank] = p;
        }
    }
    __syncthreads();
    if (mine && rank < k) {
        // the normaliser summed in slot order, so every lane of the token
        // forms the same value
        float z = 0.0f;
        for (int j = 0; j < k; ++j) z += sm.pexp[tt][j];
        ids[(size_t)t * k + rank] = e;
        gates[(size_t)t * k + rank] = p * (1.0f / z);
    }
}

// ROWS8: bf16 router rows of exactly 8 experts, read as one 16-byte vector.
// NORM: x holds h; RMSNorm(h) (eps) is written to xn and routed.
template <typename T, int EMAX, int TPW, bool ROWS8, bool NORM>
__global__ __launch_bounds__(kThreads) void router_topk_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ bias, int T_,
    int d, int E, int k, int32_t* __restrict__ ids, float* __restrict__ gates, T* __restrict__ xn,
    float eps) {
    __shared__ RouterLds<TPW, EMAX> sm;
    __shared__ float sumsq[NORM ? kWaves : 1][TPW];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    constexpr int VN = Vec<T>::N;
    const int t0 = blockIdx.x * TPW;

    // RMSNorm scale of each token (NORM only).
    float rs[TPW];
    uint4 cache[NORM ? kNormCache : 1][TPW];
    if constexpr (NORM) {
        float ss[TPW];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) ss[tt] = 0.0f;
        // slices in ascending order, the cached ones first
#pragma unroll
        for (int n = 0; n < kNormCache; ++n) {
            const int i0 = threadIdx.x * VN + n * kThreads * VN;
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                if (i0 < d && t0 + tt < T_) {
                    cache[n][tt] = *reinterpret_cast<const uint4*>(x + (size_t)(t0 + tt) * d + i0);
                    float v[VN];
                    Vec<T>::unpack(cache[n][tt], v);
#pragma unroll
                    for (int u = 0; u < VN; ++u) ss[tt] = fmaf(v[u], v[u], ss[tt]);
                }
            }
        }
        for (int i0 = threadIdx.x * VN + kNormCache * kThreads * VN; i0 < d; i0 += kThreads * VN) {
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                if (t0 + tt < T_) {
                    float v[VN];
                    Vec<T>::load(x + (size_t)(t0 + tt) * d + i0, v);
#pragma unroll
                    for (int u = 0; u < VN; ++u) ss[tt] = fmaf(v[u], v[u], ss[tt]);
                }
            }
        }
        constexpr int SH = 6 - log2_of<TPW>();
        wave_sum_split<TPW>(ss, lane);
        if ((lane & ((1 << SH) - 1)) == 0) sumsq[wave][lane >> SH] = ss[0];
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
            rs[tt] = 1.0f / sqrtf((sumsq[0][tt] + sumsq[1][tt] + sumsq[2][tt] + sumsq[3][tt]) /
                                      (float)d + eps);
    }

    float acc[TPW][EMAX];
#pragma unroll
    for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
        for (int e = 0; e < EMAX; ++e) acc[tt][e] = 0.0f;

    // Partial logits of this lane's slice at i0 for the TPW tokens in xv.
    auto accumulate = [&](int i0, float (&xv)[TPW][VN]) {
        if (ROWS8) {
#pragma unroll
            for (int u = 0; u < VN; ++u) {
                float w[8];
                Vec<T>::load(wr + (size_t)(i0 + u) * 8, w);
#pragma unroll
                for (int e = 0; e < 8; ++e)
#pragma unroll
                    for (int tt = 0; tt < TPW; ++tt) acc[tt][e] = fmaf(xv[tt][u], w[e], acc[tt][e]);
            }
        } else {
#pragma unroll
            for (int e = 0; e < EMAX; ++e) {
                if (e < E) {
#pragma unroll
                    for (int u = 0; u < VN; ++u) {
                        const float w = Vec<T>::one(wr, (size_t)(i0 + u) * E + e);
#pragma unroll
                        for (int tt = 0; tt < TPW; ++tt) acc[tt][e] = fmaf(xv[tt][u], w, acc[tt][e]);
                    }
                }
            }
        }
    };
    int i_rest = (wave * 64 + lane) * VN;  // first slice not taken from the cache
    if constexpr (NORM) {
        // (called once per cached slice, so every cache index is a constant)
        auto from_cache = [&](int i0, const uint4 (&c)[TPW]) {
            if (i0 >= d) return;
            float xv[TPW][VN];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                if (t0 + tt < T_) {
                    Vec<T>::unpack(c[tt], xv[tt]);
                    Vec<T>::scale_store(xv[tt], rs[tt], xn + (size_t)(t0 + tt) * d + i0);
                } else {
#pragma unroll
                    for (int u = 0; u < VN; ++u) xv[tt][u] = 0.0f;
                }
            }
            accumulate(i0, xv);
        };
        static_assert(kNormCache == 2, "one from_cache call per cached slice");
        from_cache(i_rest, cache[0]);
        from_cache(i_rest + kThreads * VN, cache[1]);
        i_rest += kNormCache * kThreads * VN;
    }
    for (int i0 = i_rest; i0 < d; i0 += kThreads * VN) {
        float xv[TPW][VN];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt) {
            if (t0 + tt < T_) {
                Vec<T>::load(x + (size_t)(t0 + tt) * d + i0, xv[tt]);
                if constexpr (NORM) Vec<T>::scale_store(xv[tt], rs[tt], xn + (size_t)(t0 + tt) * d + i0);
            } else {
#pragma unroll
                for (int u = 0; u < VN; ++u) xv[tt][u] = 0.0f;
            }
        }
        accumulate(i0, xv);
    }

    reduce_select<TPW, EMAX>(acc, sm, bias, t0, T_, E, k, ids, gates, lane, wave);
}

// bf16, 8 experts, d <= kLdsRows, large batches: the router matrix is
// copied to LDS once per workgroup, re-paired along the hidden dimension
// (dword (q, e) = {w[2q][e], w[2q+1][e]}), and each workgroup walks token
// groups g = blockIdx.x, blockIdx.x + gridDim.x, ... with every 16-byte slice
// of a group's rows loaded at once and the next group's rows in flight while
// the current group is reduced.  The logits are taken with
// v_dot2c_f32_bf16 -- two bf16 products added to an fp32 accumulator per
// instruction, straight from the packed pairs in x and in LDS -- which halves
// the instruction count of the fmaf form and needs no unpacking; at these
// batch sizes the router is otherwise bound by those instructions (fp32
// logits either way; the slices per thread and the reductions are as in
// router_topk_kernel).
constexpr int kLdsRows = 4096;
constexpr int kLdsMinTokens = 768;  // below this the one-group-per-workgroup kernel is used
constexpr int kLdsWgsPerCu = 2;     // resident workgroups per CU (LDS: 66 KiB each)

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b),
                                           c, false);
}
__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int TPW, bool NORM>
__global__ __launch_bounds__(kThreads, 2) void router_lds_kernel(
    const bf16* __restrict__ x, const bf16* __restrict__ wr, const float* __restrict__ bias, int T_,
    int d, int k, int32_t* __restrict__ ids, float* __restrict__ gates, bf16* __restrict__ xn,
    float eps) {
    constexpr int VN = 8;                          // bf16 per 16-byte slice
    constexpr int NS = kLdsRows / (kThreads * VN);  // slices per thread
    // wl[2 q + h]: the four dwords {w[2q][e], w[2q+1][e]} of experts 4h .. 4h+3
    __shared__ uint4 wl[kLdsRows];
    __shared__ RouterLds<TPW, 8> sm;
    __shared__ float sumsq[NORM ? kWaves : 1][TPW];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int groups = (T_ + TPW - 1) / TPW;

    auto load_group = [&](int g, uint4 (&q)[TPW][NS]) {
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            const int i0 = (threadIdx.x + kThreads * sl) * VN;
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const int t = g * TPW + tt;
                q[tt][sl] = (g < groups && t < T_ && i0 < d)
                                ? *reinterpret_cast<const uint4*>(x + (size_t)t * d + i0)
                                : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };

    // the first group's rows are in flight while the router matrix is copied
    uint4 xq[TPW][NS];
    load_group(blockIdx.x, xq);
    for (int q = threadIdx.x; 2 * q < d; q += kThreads) {
        const uint4 r0 = reinterpret_cast<const uint4*>(wr)[2 * q];
        const uint4 r1 = reinterpret_cast<const uint4*>(wr)[2 * q + 1];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t a0 = word(r0, 2 * h), a1 = word(r0, 2 * h + 1);  // experts 4h..4h+3 of row 2q
            const uint32_t b0 = word(r1, 2 * h), b1 = word(r1, 2 * h + 1);  // and of row 2q+1
            wl[2 * q + h] = make_uint4(__builtin_amdgcn_perm(b0, a0, 0x05040100u),
                                       __builtin_amdgcn_perm(b0, a0, 0x07060302u),
                                       __builtin_amdgcn_perm(b1, a1, 0x05040100u),
                                       __builtin_amdgcn_perm(b1, a1, 0x07060302u));
        }
    }
    __syncthreads();
    for (int g = blockIdx.x; g < groups; g += gridDim.x) {
        uint4 xnext[TPW][NS];
        load_group(g + gridDim.x, xnext);
        const int t0 = g * TPW;
        if constexpr (NORM) {
            // sum of squares in the order of rmsnorm_kernel: this thread's
            // slices ascending, fmaf element by element, then the wave
            // butterfly and the 4 waves in order (the same bits as
            // moe_rmsnorm); then each slice scaled, rounded once, stored as
            // the layer input, and routed from those rounded values
            float ss[TPW];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) ss[tt] = 0.0f;
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) {
                const int i0 = (threadIdx.x + kThreads * sl) * VN;
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    if (i0 < d && t0 + tt < T_) {
                        float v[VN];
                        Vec<bf16>::unpack(xq[tt][sl], v);
#pragma unroll
                        for (int u = 0; u < VN; ++u) ss[tt] = fmaf(v[u], v[u], ss[tt]);
                    }
                }
            }
            constexpr int SH = 6 - log2_of<TPW>();
            wave_sum_split<TPW>(ss, lane);
            if ((lane & ((1 << SH) - 1)) == 0) sumsq[wave][lane >> SH] = ss[0];
            __syncthreads();
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                const float r = 1.0f / sqrtf((sumsq[0][tt] + sumsq[1][tt] + sumsq[2][tt] +
                                              sumsq[3][tt]) / (float)d + eps);
#pragma unroll
                for (int sl = 0; sl < NS; ++sl) {
                    const int i0 = (threadIdx.x + kThreads * sl) * VN;
                    if (i0 < d && t0 + tt < T_) {
                        float v[VN];
                        Vec<bf16>::scale_store_words(xq[tt][sl], v, r, xn + (size_t)(t0 + tt) * d + i0);
                    }
                }
            }
        }
        float acc[TPW][8];
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[tt][e] = 0.0f;
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) {
            const int i0 = (threadIdx.x + kThreads * sl) * VN;
            if (i0 >= d) break;
#pragma unroll
            for (int q = 0; q < VN / 2; ++q) {
                const uint4 w0 = wl[i0 + 2 * q];      // pair i0/2 + q, experts 0..3
                const uint4 w1 = wl[i0 + 2 * q + 1];  // experts 4..7
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt) {
                    const uint32_t xp = word(xq[tt][sl], q);
                    acc[tt][0] = dot2_bf16(xp, w0.x, acc[tt][0]);
                    acc[tt][1] = dot2_bf16(xp, w0.y, acc[tt][1]);
                    acc[tt][2] = dot2_bf16(xp, w0.z, acc[tt][2]);
                    acc[tt][3] = dot2_bf16(xp, w0.w, acc[tt][3]);
                    acc[tt][4] = dot2_bf16(xp, w1.x, acc[tt][4]);
                    acc[tt][5] = dot2_bf16(xp, w1.y, acc[tt][5]);
                    acc[tt][6] = dot2_bf16(xp, w1.z, acc[tt][6]);
                    acc[tt][7] = dot2_bf16(xp, w1.w, acc[tt][7]);
                }
            }
        }
        reduce_select<TPW, 8>(acc, sm, bias, t0, T_, 8, k, ids, gates, lane, wave);
#pragma unroll
        for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
            for (int sl = 0; sl < NS; ++sl) xq[tt][sl] = xnext[tt][sl];
    }
}

// Compute units of the current device (queried once per device).
int device_cus() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1)
            c = 256;
        cached[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <int TPW>
hipError_t launch_lds(const void* x, const void* wr, const float* bias, int T_, int d, int k,
                      int32_t* ids, float* gates, void* xn, float eps, int wgs_per_cu,
                      hipStream_t stream) {
    const int groups = (T_ + TPW - 1) / TPW;
    int blocks = device_cus() * wgs_per_cu;
    if (blocks > groups) blocks = groups;
    if (xn != nullptr)
        hipLaunchKernelGGL((router_lds_kernel<TPW, true>), dim3(blocks), dim3(kThreads), 0, stream,
                           reinterpret_cast<const bf16*>(x), reinterpret_cast<const bf16*>(wr), bias,
                           T_, d, k, ids, gates, reinterpret_cast<bf16*>(xn), eps);
    else
        hipLaunchKernelGGL((router_lds_kernel<TPW, false>), dim3(blocks), dim3(kThreads), 0, stream,
                           reinterpret_cast<const bf16*>(x), reinterpret_cast<const bf16*>(wr), bias,
                           T_, d, k, ids, gates, static_cast<bf16*>(nullptr), 0.0f);
    return hipGetLastError();
}

template <typename T, int EMAX, int TPW, bool ROWS8>
hipError_t launch_t(const void* x, const void* wr, const float* bias, int T_, int d, int E, int k,
                    int32_t* ids, float* gates, void* xn, float eps, hipStream_t stream) {
    const int blocks = (T_ + TPW - 1) / TPW;
    if (xn != nullptr)
        hipLaunchKernelGGL((router_topk_kernel<T, EMAX, TPW, ROWS8, true>), dim3(blocks),
                           dim3(kThreads), 0, stream, reinterpret_cast<const T*>(x),
                           reinterpret_cast<const T*>(wr), bias, T_, d, E, k, ids, gates,
                           reinterpret_cast<T*>(xn), eps);
    else
        hipLaunchKernelGGL((router_topk_kernel<T, EMAX, TPW, ROWS8, false>), dim3(blocks),
                           dim3(kThreads), 0, stream, reinterpret_cast<const T*>(x),
                           reinterpret_cast<const T*>(wr), bias, T_, d, E, k, ids, gates,
                           static_cast<T*>(nullptr), 0.0f);
    return hipGetLastError();
}

template <typename T>
hipError_t dispatch_e(const void* x, const void* wr, const float* bias, int T_, int d, int E,
                      int k, int32_t* ids, float* gates, void* xn, float eps, hipStream_t stream) {
    // Larger batches share each router row load among more tokens of a
    // workgroup (measured on MI355X at d = 4096: 1 token per workgroup is
    // fastest up to a few hundred tokens, 8 from a few thousand).
    const bool big = T_ > 1024;
    if constexpr (sizeof(T) == 2) {
        if (E == 8 && d <= kLdsRows && T_ > kLdsMinTokens) {
            // (the RMSNorm form holds more per token: 4 tokens per group)
            if (T_ > 2048 && xn == nullptr)
                return launch_lds<8>(x, wr, bias, T_, d, k, ids, gates, xn, eps, kLdsWgsPerCu, stream);
            return launch_lds<4>(x, wr, bias, T_, d, k, ids, gates, xn, eps, kLdsWgsPerCu, stream);
        }
        if (E == 8) {
            // (the fused RMSNorm keeps its rows in registers: at most 4 tokens)
            if (T_ > 2048 && xn == nullptr)
                return launch_t<T, 8, 8, true>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
            if (T_ > 768) return launch_t<T, 8, 4, true>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
            if (T_ > 384) return launch_t<T, 8, 2, true>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
            return launch_t<T, 8, 1, true>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
        }
    }
    if (E <= 8) {
        if (big) return launch_t<T, 8, 4, false>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
        return launch_t<T, 8, 1, false>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
    }
    if (E <= 16) return launch_t<T, 16, 2, false>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
    if (E <= 32) return launch_t<T, 32, 1, false>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
    return launch_t<T, 64, 1, false>(x, wr, bias, T_, d, E, k, ids, gates, xn, eps, stream);
}

}  // namespace

hipError_t launch_router_topk(int dtype, const void* x, const void* w_router, const float* bias,
                              int T, int d, int E, int k, int32_t* ids, float* gates, void* xn,
                              float eps, hipStream_t stream) {
    if (dtype == 0) return dispatch_e<bf16>(x, w_router, bias, T, d, E, k, ids, gates, xn, eps, stream);
    return dispatch_e<float>(x, w_router, bias, T, d, E, k, ids, gates, xn, eps, stream);
}

}  // namespace moe
