// route_permute.hip -- group the (token, pick) assignments by expert.
//
// Mixtral of Experts (wikillm.com card, "Method"): the layer is applied to a
// whole batch at once, grouped by expert, with no capacity limit, so every
// token reaches exactly k experts ("Pitfalls": no capacity limit or token
// dropping).  Here the grouping is explicit:
//   counts[e]   assignments routed to expert e
//   offsets[e]  exclusive prefix sum of counts (offsets[E] = T*k)
//   slot_row[a] grouped row of assignment a = t*k + j
//   row_token[r] token of grouped row r
// Rows of one expert are contiguous and in ascending (token, pick) order, so
// the permutation is stable and deterministic (no atomics).
//
// route_scan_kernel is one workgroup of 16 wavefronts.  Each wave owns a
// contiguous run of 64-assignment chunks.  Pass 1 counts, per expert, with
// one ballot per expert per chunk; the per-wave counts are scanned in LDS;
// pass 2 walks the same chunks again and gives each assignment its row as
// (expert base + wave base + rank among earlier equal lanes).
//
// gather_rows_kernel then copies x[row_token[r]] into x_perm[r] with 16-byte
// loads and stores, one row per wave iteration, so every read of a token row
// is a contiguous, coalesced stream.
#include "common.h"

namespace moe {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kBatch = 8;  // chunks of 64 ids loaded together per wave

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_row,
    int32_t* __restrict__ row_token) {
    __shared__ int wave_count[kScanWaves][64];
    __shared__ int wave_base[kScanWaves][64];
    __shared__ int expert_base[65];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int nchunks = (R + 63) / 64;
    const int per_wave = (nchunks + kScanWaves - 1) / kScanWaves;
    const int c0 = wave * per_wave;
    const int c1 = min(c0 + per_wave, nchunks);

    // Pass 1: lane e accumulates this wave's count for expert e.  The ids of
    // up to kBatch chunks are loaded together, so their latencies overlap.
    int mine = 0;
    for (int cb = c0; cb < c1; cb += kBatch) {
        int eb[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int a = (cb + u) * 64 + lane;
            eb[u] = (cb + u < c1 && a < R) ? ids[a] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (cb + u >= c1) break;  // wave-uniform
            for (int ex = 0; ex < E; ++ex) {
                const uint64_t m = __ballot(eb[u] == ex);
                if (lane == ex) mine += __popcll(m);
            }
        }
    }
    wave_count[wave][lane] = mine;
    __syncthreads();

    // Per expert: exclusive scan over waves; then over experts.
    if (threadIdx.x < 64) {
        const int e = threadIdx.x;
        int run = 0;
        for (int w = 0; w < kScanWaves; ++w) {
            wave_base[w][e] = run;
            run += (e < E) ? wave_count[w][e] : 0;
        }
        // exclusive scan of the totals across the 64 lanes of wave 0
        int incl = run;
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (e >= off) incl += v;
        }
        const int excl = incl - run;
        if (e < E) {
            expert_base[e] = excl;
            counts[e] = run;
            offsets[e] = excl;
        }
        if (e == E - 1) {
            expert_base[E] = incl;
            offsets[E] = incl;
        }
    }
    __syncthreads();

    // Pass 2: lane ex keeps the next free row of expert ex for this wave.
    int next = (lane < E) ? expert_base[lane] + wave_base[wave][lane] : 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int cb = c0; cb < c1; cb += kBatch) {
        int eb[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int a = (cb + u) * 64 + lane;
            eb[u] = (cb + u < c1 && a < R) ? ids[a] : -1;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            if (cb + u >= c1) break;  // wave-uniform
            const int a = (cb + u) * 64 + lane;
            const int e = eb[u];
            int row = -1;
            for (int ex = 0; ex < E; ++ex) {
                const uint64_t m = __ballot(e == ex);
                const int base = __shfl(next, ex, 64);
                if (e == ex) row = base + __popcll(m & below);
                if (lane == ex) next += __popcll(m);
            }
            if (e >= 0) {
                slot_row[a] = row;
                row_token[row] = a / k;
            }
        }
    }
}

template <int VEC_BYTES>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int32_t* __restrict__ row_token,
                                                          int R, int vec_per_row,
                                                          uint4* __restrict__ x_perm) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    for (int r = blockIdx.x * 4 + wave; r < R; r += gridDim.x * 4) {
        const int t = row_token[r];
        const uint4* src = x + (size_t)t * vec_per_row;
        uint4* dst = x_perm + (size_t)r * vec_per_row;
        for (int v = lane; v < vec_per_row; v += 64) dst[v] = src[v];
    }
}

// The same gather into the K-blocked layout of the 256-row tile GEMM:
// element (r, i) of x_perm [R, d] at ((i / 32) * R + r) * 32 + i % 32, so one
// 32-wide K block of consecutive rows is one contiguous run.  Thread unit u =
// (block, row, 16-byte piece) with the piece fastest: writes are contiguous.
__global__ __launch_bounds__(256) void gather_rows_kb_kernel(const uint4* __restrict__ x,
                                                             const int32_t* __restrict__ row_token,
                                                             int R, int vec_per_row,
                                                             uint4* __restrict__ x_perm) {
    const size_t units = (size_t)R * vec_per_row;
    for (size_t u = (size_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (size_t)gridDim.x * 256) {
        const int piece = (int)(u & 3);
        const size_t rb = u >> 2;
        const int r = (int)(rb % (size_t)R);
        const int b = (int)(rb / (size_t)R);
        const int t = row_token[r];
        x_perm[u] = x[(size_t)t * vec_per_row + 4 * b + piece];
    }
}

__global__ __launch_bounds__(256) void sum_splits_kernel(const float4* __restrict__ y, int splits,
                                                         size_t n4, float4* __restrict__ out) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (size_t)gridDim.x * 256) {
        float4 s = y[i];
        for (int p = 1; p < splits; ++p) {
            const float4 v = y[(size_t)p * n4 + i];
            s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
        }
        out[i] = s;
    }
}

}  // namespace

hipError_t launch_route_scan(const int32_t* ids, int T, int k, int E, int32_t* counts,
                             int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                             hipStream_t stream) {
    hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, ids, T * k, k, E,
                       counts, offsets, slot_row, row_token);
    return hipGetLastError();
}

hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* row_token, int R, int d,
                              int kb, void* x_perm, hipStream_t stream) {
    const int esize = dtype == 0 ? 2 : 4;
    const int vec_per_row = d * esize / 16;
    if (kb) {
        // bf16 only: 32-element blocks are 4 16-byte pieces (d is a multiple of 64)
        const size_t units = (size_t)R * vec_per_row;
        size_t blocks = (units + 255) / 256;
        if (blocks > 16384) blocks = 16384;
        if (blocks < 1) blocks = 1;
        hipLaunchKernelGGL(gather_rows_kb_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                           reinterpret_cast<const uint4*>(x), row_token, R, vec_per_row,
                           reinterpret_cast<uint4*>(x_perm));
        return hipGetLastError();
    }
    int blocks = (R + 3) / 4;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(gather_rows_kernel<16>, dim3(blocks), dim3(256), 0, stream,
                       reinterpret_cast<const uint4*>(x), row_token, R, vec_per_row,
                       reinterpret_cast<uint4*>(x_perm));
    return hipGetLastError();
}

hipError_t launch_sum_splits(const float* y, int splits, int R, int d, float* y_out,
                             hipStream_t stream) {
    const size_t n4 = (size_t)R * d / 4;
    size_t blocks = (n4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       reinterpret_cast<const float4*>(y), splits, n4,
                       reinterpret_cast<float4*>(y_out));
    return hipGetLastError();
}

}  // namespace moe
