// common.h -- device types, conversions and launcher declarations shared by
// the kernels of libmoe_ffn (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Widening bf16 -> fp32 is exact: the bf16 bits are the high half of the fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// SiLU(z) = z * sigmoid(z), fp32, with the sigmoid's reciprocal taken by
// v_rcp_f32 (1 ulp) rather than an IEEE division (about ten VALU instructions
// per value in the GEMM 1 epilogues); h is rounded to bf16 right after, or
// kept in fp32 within 1 ulp.  Large |z| keep their limits: exp(-z) = inf
// gives z * 0 = -0, exp(-z) = 0 gives z.
__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// Kernel launchers.  Each returns the hipGetLastError() of its launch(es).
// dtype: 0 = bf16, 1 = fp32 (same codes as moe_dtype_t).

// xn: when non-null, x holds h and the router writes x = RMSNorm(h) (eps,
// unit gain, the same bits as launch_rmsnorm) to xn and routes that.
hipError_t launch_router_topk(int dtype, const void* x, const void* w_router, const float* bias,
                              int T, int d, int E, int k, int32_t* ids, float* gates, void* xn,
                              float eps, hipStream_t stream);

// scratch: route_scan_scratch_bytes(T * k, E) bytes (0: may be null)
size_t route_scan_scratch_bytes(int R, int E);
hipError_t launch_route_scan(const int32_t* ids, int T, int k, int E, int32_t* counts,
                             int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                             int32_t* scratch, hipStream_t stream);

// kb: write x_perm in the K-blocked layout of the 256-row tile GEMM (bf16)
hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* row_token, int R, int d,
                              int kb, void* x_perm, hipStream_t stream);

// Grouped GEMM 1 with the SwiGLU epilogue: for each grouped row r of expert e,
// h[r,:] = SiLU(x_perm[r,:] . w1[e]) * (x_perm[r,:] . w3[e]).
hipError_t launch_gemm1_swiglu_bf16(int variant, const void* x_perm, const void* w1,
                                    const void* w3, const int32_t* offsets, int R, int E, int d,
                                    int f, void* h, hipStream_t stream);
hipError_t launch_gemm1_swiglu_f32(const void* x_perm, const void* w1, const void* w3,
                                   const int32_t* offsets, int R, int E, int d, int f, void* h,
                                   hipStream_t stream);

// Grouped GEMM 2: y[s][r,:] = h[r, Ks] . w2[e][Ks, :] over the s-th of
// `splits` equal slices Ks of the contraction; fp32 partials.
hipError_t launch_gemm2_bf16(int variant, const void* h, const void* w2, const int32_t* offsets,
                             int R, int E, int f, int d, int splits, float* y,
                             hipStream_t stream);
hipError_t launch_gemm2_f32(const void* h, const void* w2, const int32_t* offsets, int R, int E,
                            int f, int d, float* y, hipStream_t stream);

// The same two contractions for batches with few rows per expert: weights are
// streamed from HBM into registers (row tiles of up to 64 rows, in 16-row
// fragments sized per tile on the device; 128-column slabs).
// (reads the token rows of x through row_token: no gathered copy is needed;
// k_waves = 1, 2 or 4 waves split K for each 128-column slab, with 4, 2 or
// 1 slabs per workgroup)
hipError_t launch_gemm1_swiglu_stream(const void* x, const int32_t* row_token, const void* w1,
                                      const void* w3, const int32_t* offsets, int R, int E, int d,
                                      int f, int k_waves, void* h, hipStream_t stream);
hipError_t launch_gemm2_stream(const void* h, const void* w2, const int32_t* offsets, int R, int E,
                               int f, int d, int splits, float* y, hipStream_t stream);

// The same two contractions for batches with many rows per expert: 256x256
// macro tiles staged through LDS.  In GEMM 2 each XCD's last, partial round
// of tiles may be cut into K pieces whose fp32 partial sums go to `partials`
// (tile_partials_bytes(R, E, d, f) bytes of scratch, also used by GEMM 1 for
// a small header) and are summed, in piece order, by a second kernel that
// stores y; launch_gemm2_tile makes both launches.
// kb: A (x_perm) and the h output in the K-blocked layout
size_t tile_partials_bytes(int R, int E, int d, int f);
// nt_weights: mark the w1/w3 DMA nontemporal (each weight panel read by one
// row tile: at up to ~192 rows per expert; GEMM 2's weight DMA always is).
hipError_t launch_gemm1_swiglu_tile(const void* x_perm, const void* w1, const void* w3,
                                    const int32_t* offsets, int R, int E, int d, int f, int kb,
                                    float* partials, bool nt_weights, void* h, hipStream_t stream);
// kb: A (h) in the K-blocked layout; y [R, d] fp32 (one slice)
hipError_t launch_gemm2_tile(const void* h, const void* w2, const int32_t* offsets, int R, int E,
                             int f, int d, int kb, float* partials, float* y, hipStream_t stream);

// out[t,:] = (residual[t,:] +) sum_j gates[t,j] * sum_s y[s][slot_row[t*k+j], :]
hipError_t launch_combine(int dtype, const float* y, int splits, const float* gates,
                          const int32_t* slot_row, const void* residual, int T, int d, int k, int R,
                          void* out, hipStream_t stream);

// y_out[r,:] = sum_s y[s][r,:]
hipError_t launch_sum_splits(const float* y, int splits, int R, int d, float* y_out,
                             hipStream_t stream);

hipError_t launch_rmsnorm(int dtype, const void* h, void* x, int T, int d, float eps,
                          hipStream_t stream);

// Streaming read of `bytes` (a multiple of 16) from buf; XOR fold to *sink.
hipError_t launch_read_probe(const void* buf, size_t bytes, int blocks, uint32_t* sink,
                             hipStream_t stream);

// bf16 MFMA work on operands read once from ops (bytes, a multiple of 16):
// `blocks` workgroups of 4 waves, each wave iters x 128 v_mfma_f32_16x16x32_bf16.
// clocks (optional): per workgroup {shader cycles, 100 MHz ticks}.
hipError_t launch_mfma_probe(const void* ops, size_t bytes, int iters, int blocks, uint32_t* sink,
                             unsigned long long* clocks, hipStream_t stream);

// Tile shapes of the bf16 grouped GEMMs, chosen by the host per call.
enum GemmVariant { GEMM_LARGE_M = 0, GEMM_SMALL_M = 1, GEMM_STREAM = 2, GEMM_TILE256 = 3 };
int gemm_bm(int variant);      // rows per tile
int gemm1_bn(int variant);     // h columns per tile
int gemm2_bn(int variant);     // y columns per tile

}  // namespace moe
