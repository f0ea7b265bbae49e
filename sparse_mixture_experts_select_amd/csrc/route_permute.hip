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
// Past kScanSingleMax assignments the same two passes run over many
// workgroups instead of one: route_count_kernel writes each workgroup's
// per-expert counts of its contiguous block of assignments; route_place_kernel
// reads all of them, forms the expert offsets and its block's base per expert
// (the counts of the blocks before it), and ranks its block's assignments
// exactly as the single-workgroup kernel does, so the grouping is identical.
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
// above this many assignments the multi-workgroup form runs
constexpr int kScanSingleMax = 4096;

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

constexpr int kBlockThreads = 256;
constexpr int kBlockWaves = kBlockThreads / 64;
constexpr int kBlockChunks = 4;                            // chunks of 64 per wave
constexpr int kBlockIds = kBlockWaves * kBlockChunks * 64;  // assignments per workgroup

// Per-expert counts of workgroup b's assignments [b * kBlockIds, ...).
__global__ __launch_bounds__(kBlockThreads) void route_count_kernel(const int32_t* __restrict__ ids,
                                                                     int R, int E,
                                                                     int32_t* __restrict__ blk_counts) {
    __shared__ int wave_count[kBlockWaves][64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int c0 = blockIdx.x * kBlockWaves * kBlockChunks + wave * kBlockChunks;
    int eb[kBlockChunks];
#pragma unroll
    for (int u = 0; u < kBlockChunks; ++u) {
        const int a = (c0 + u) * 64 + lane;
        eb[u] = a < R ? ids[a] : -1;
    }
    int mine = 0;
#pragma unroll
    for (int u = 0; u < kBlockChunks; ++u)
        for (int ex = 0; ex < E; ++ex) {
            const uint64_t m = __ballot(eb[u] == ex);
            if (lane == ex) mine += __popcll(m);
        }
    wave_count[wave][lane] = mine;
    __syncthreads();
    if (threadIdx.x < 64 && threadIdx.x < E) {
        int tot = 0;
#pragma unroll
        for (int w = 0; w < kBlockWaves; ++w) tot += wave_count[w][threadIdx.x];
        blk_counts[(size_t)blockIdx.x * E + threadIdx.x] = tot;
    }
}

// Rows of workgroup b's assignments: expert base + the counts of the blocks
// before b + the wave's base in the block + the rank among earlier equal
// lanes.  Workgroup 0 also writes counts and offsets.
__global__ __launch_bounds__(kBlockThreads) void route_place_kernel(
    const int32_t* __restrict__ ids, int R, int k, int E, int nblk,
    const int32_t* __restrict__ blk_counts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_row, int32_t* __restrict__ row_token) {
    __shared__ int wave_count[kBlockWaves][64];
    __shared__ int base_s[64];
    __shared__ int total_s[64];
    __shared__ int before_s[64];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    if (threadIdx.x < 64) {
        total_s[threadIdx.x] = 0;
        before_s[threadIdx.x] = 0;
    }
    __syncthreads();
    // every block's counts, summed per expert (integer sums: any order)
    for (int i = threadIdx.x; i < nblk * E; i += kBlockThreads) {
        const int b = i / E;
        const int e = i - b * E;
        const int c = blk_counts[i];
        atomicAdd(&total_s[e], c);
        if (b < (int)blockIdx.x) atomicAdd(&before_s[e], c);
    }
    const int c0 = blockIdx.x * kBlockWaves * kBlockChunks + wave * kBlockChunks;
    int eb[kBlockChunks];
#pragma unroll
    for (int u = 0; u < kBlockChunks; ++u) {
        const int a = (c0 + u) * 64 + lane;
        eb[u] = a < R ? ids[a] : -1;
    }
    int mine = 0;
#pragma unroll
    for (int u = 0; u < kBlockChunks; ++u)
        for (int ex = 0; ex < E; ++ex) {
            const uint64_t m = __ballot(eb[u] == ex);
            if (lane == ex) mine += __popcll(m);
        }
    wave_count[wave][lane] = mine;
    __syncthreads();
    if (wave == 0) {
        // lane e: total of expert e and the part before this block
        const int total = lane < E ? total_s[lane] : 0;
        const int before = lane < E ? before_s[lane] : 0;
        int incl = total;
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        const int excl = incl - total;
        if (lane < E) base_s[lane] = excl + before;
        if (blockIdx.x == 0) {
            if (lane < E) {
                counts[lane] = total;
                offsets[lane] = excl;
            }
            if (lane == E - 1) offsets[E] = incl;
        }
    }
    __syncthreads();
    // this wave's base per expert: block base + the waves before it
    int next = 0;
    if (lane < E) {
        next = base_s[lane];
        for (int w = 0; w < wave; ++w) next += wave_count[w][lane];
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int u = 0; u < kBlockChunks; ++u) {
        const int a = (c0 + u) * 64 + lane;
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
// The tile path keeps x_perm under 2 GiB, so unit numbers fit in 32 bits.
__global__ __launch_bounds__(256) void gather_rows_kb_kernel(const uint4* __restrict__ x,
                                                             const int32_t* __restrict__ row_token,
                                                             int R, int vec_per_row,
                                                             uint4* __restrict__ x_perm) {
    const uint32_t units = (uint32_t)R * (uint32_t)vec_per_row;
    const uint32_t ur = (uint32_t)R;
    for (uint32_t u = blockIdx.x * 256u + threadIdx.x; u < units; u += gridDim.x * 256u) {
        const uint32_t rb = u >> 2;
        const uint32_t b = rb / ur;
        const uint32_t r = rb - b * ur;
        const int t = row_token[r];
        x_perm[u] = x[(size_t)t * vec_per_row + 4 * b + (u & 3)];
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

size_t route_scan_scratch_bytes(int R, int E) {
    if (R <= kScanSingleMax) return 0;
    return (size_t)((R + kBlockIds - 1) / kBlockIds) * E * sizeof(int32_t);
}

hipError_t launch_route_scan(const int32_t* ids, int T, int k, int E, int32_t* counts,
                             int32_t* offsets, int32_t* slot_row, int32_t* row_token,
                             int32_t* scratch, hipStream_t stream) {
    const int R = T * k;
    if (R <= kScanSingleMax) {
        hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), 0, stream, ids, R, k, E,
                           counts, offsets, slot_row, row_token);
        return hipGetLastError();
    }
    const int nblk = (R + kBlockIds - 1) / kBlockIds;
    hipLaunchKernelGGL(route_count_kernel, dim3(nblk), dim3(kBlockThreads), 0, stream, ids, R, E,
                       scratch);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(route_place_kernel, dim3(nblk), dim3(kBlockThreads), 0, stream, ids, R, k, E,
                       nblk, scratch, counts, offsets, slot_row, row_token);
    return hipGetLastError();
}

hipError_t launch_gather_rows(int dtype, const void* x, const int32_t* row_token, int R, int d,
                              int kb, void* x_perm, hipStream_t stream) {
    const int esize = dtype == 0 ? 2 : 4;
    const int vec_per_row = d * esize / 16;
    if (kb) {
        // bf16 only: 32-element blocks are 4 16-byte pieces (d is a multiple
        // of 64); the caller keeps R * d * 2 bytes under 2 GiB
        const size_t units = (size_t)R * vec_per_row;
        if (units >= ((size_t)1 << 31)) return hipErrorInvalidValue;
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
    hipLaunchKernelGGL(gather_rows_kernel, dim3(blocks), dim3(256), 0, stream,
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
