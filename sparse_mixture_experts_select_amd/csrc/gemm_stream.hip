// gemm_stream.hip -- the expert contractions for batches with few rows per
// expert (decode), where the time is the HBM stream of the expert weights.
//
// Same products as gemm_bf16.hip (Mixtral of Experts, wikillm.com card,
// "Method", SwiGLU pseudocode): per expert e, GEMM 1 h = SiLU(X_e.w1[e]) *
// (X_e.w3[e]) and GEMM 2 y = h_e.w2[e], over the expert's grouped rows.
//
// Work unit: (expert, row tile of up to 64 rows, 128-column slab(s), K
// slice).  Each tile takes MF = 1, 2 or 4 fragments of 16 rows by its own
// row count (read from the device-side offsets), so an expert with up to 64
// rows reads its weights once, and each weight block loaded feeds MF MFMAs.
// Workgroups of 4 wavefronts in three shapes, by KW, the number of waves
// that split the slice's K range for one slab:
//   KW = 1: 4 adjacent slabs, one per wave, each over the slice's whole K
//           range (no reduction): every w row is read as 512 contiguous
//           columns per workgroup (GEMM 1, and GEMM 2 with its K range cut
//           into slices across workgroups);
//   KW = 2: 2 adjacent slabs, two waves each on the two halves of K;
//   KW = 4: one slab, the 4 waves on 4 contiguous quarters of K.
// With KW > 1 (GEMM 1 when only a few experts hold rows, so that enough
// workgroups stream) tiles hold 16 rows and the waves of a slab add their
// partial sums in LDS once at the end.
// GEMM 1 reads its A rows straight from the token rows of x through the
// row -> token map (no gathered copy of x is made on this path).
// Each wavefront streams its weight rows straight from HBM into registers:
// per 32-row K step, lane (g = lane/16, j = lane%16) loads the 8x8 block
// (rows 8g..8g+7 of the step, columns 8j..8j+7 of the slab) with eight
// 16-byte loads -- every load instruction reads four 256-byte row segments --
// and transposes it in registers with byte permutes into the B operands of 8
// v_mfma_f32_16x16x32_bf16 (fragment c holds columns 8j+c).  The A operand
// (16 rows x 32 k of X, L2-resident) is one 16-byte load per lane and
// fragment.  Weights never pass through LDS.  The next K step's weights are
// always in flight while a step computes: GEMM 1 loads w1 of step kt+1 while
// the w3 half of step kt computes and w3 of step kt+1 while the w1 half of
// step kt+1 computes (the same registers as a loop without prefetch); GEMM 2
// (one matrix) keeps two steps of w2 in registers.  Loads are unconditional:
// rows past the expert's last row and columns past N read clamped, valid
// addresses, and only feed output rows / columns that are never stored.
//
// Epilogue: lane holds rows 4g..4g+3 of each fragment and the 8 consecutive
// columns 8j..8j+7 of its slab, so each row is written with one 16-byte
// (bf16 h) or two 16-byte (fp32 y) stores.  GEMM 1 applies SiLU(a)*b; GEMM 2
// writes fp32 partials of its K slice, summed later in a fixed order.
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kFrag = 16;      // rows per fragment
constexpr int kMaxFrags = 4;   // fragments per row tile
constexpr int kSlab = 128;     // columns per slab
constexpr int kKS = 32;        // k per step

// A weight load: each weight byte is read once per launch (one workgroup per
// expert, slab and K slice), so it is marked nontemporal -- a streaming read
// that HBM serves at 7.2 TB/s where the same loads without the hint reach
// 6.4 TB/s (4 GiB read on MI355X).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const bf16* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint32_t dw(const uint4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Column c (0..7) of an 8x8 bf16 block held as 8 row vectors.
__device__ __forceinline__ bf16x8 block_column(const uint4 (&v)[8], int c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const int q = c >> 1;
    uint4 o;
    o.x = __builtin_amdgcn_perm(dw(v[1], q), dw(v[0], q), sel);
    o.y = __builtin_amdgcn_perm(dw(v[3], q), dw(v[2], q), sel);
    o.z = __builtin_amdgcn_perm(dw(v[5], q), dw(v[4], q), sel);
    o.w = __builtin_amdgcn_perm(dw(v[7], q), dw(v[6], q), sel);
    return __builtin_bit_cast(bf16x8, o);
}

// One row tile: rows row0 .. row0 + 16*MF - 1 (those at or past row_end are
// computed on clamped addresses and not stored) of the expert whose weights
// start at B0/B1 + b_base, against the workgroup's slab(s), over K steps
// [s0, s1) of the split.
// a_rows: when non-null, grouped row r of A is row a_rows[r] of the A matrix
// (GEMM 1 reading the token rows of x directly, with no gathered copy).
template <bool DUAL, int KW, int MF>
__device__ __forceinline__ void stream_tile(const bf16* __restrict__ A,
                                            const int32_t* __restrict__ a_rows,
                                            const bf16* __restrict__ B0,
                                            const bf16* __restrict__ B1, void* __restrict__ C,
                                            size_t b_base, int row0, int row_end, int n_tile,
                                            int split, int s0, int s1, int R, int K, int N,
                                            floatx4 (*red)[64]) {
    constexpr int NMAT = DUAL ? 2 : 1;
    constexpr int TILE_N = (4 / KW) * kSlab;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int j = lane & 15;
    const int kpart = wave % KW;  // this wave's part of K (KW > 1)
    const int slab = wave / KW;   // this wave's slab in the workgroup

    // K range: the split's slice (with KW > 1 this wave's part of it).
    int k0 = s0, k1 = s1;
    if (KW > 1) {
        const int q = (s1 - s0 + KW - 1) / KW;
        k0 = min(s0 + kpart * q, s1);
        k1 = min(k0 + q, s1);
    }

    // A fragment f: rows row0 + 16 f + j (past the expert: its last row, a
    // valid address feeding only rows that are never stored).
    const bf16* a_ptr[MF];
#pragma unroll
    for (int f = 0; f < MF; ++f) {
        const int arow = min(row0 + kFrag * f + j, row_end - 1);
        a_ptr[f] = A + (size_t)(a_rows ? a_rows[arow] : arow) * K + 8 * g;
    }
    const int col = n_tile * TILE_N + slab * kSlab + 8 * j;
    const bool b_ok = col < N;
    const size_t b_off = b_base + (size_t)(8 * g) * N + (b_ok ? col : 0);
    const bf16* b_ptr[NMAT];
    b_ptr[0] = B0 + b_off;
    if (DUAL) b_ptr[NMAT - 1] = B1 + b_off;

    floatx4 acc[MF][NMAT][8];
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int c = 0; c < 8; ++c) acc[f][m][c] = floatx4{0.f, 0.f, 0.f, 0.f};

    auto load_a = [&](int kt, uint4 (&a)[MF]) {
#pragma unroll
        for (int f = 0; f < MF; ++f) a[f] = *reinterpret_cast<const uint4*>(a_ptr[f] + (size_t)kt * kKS);
    };
    auto load_b = [&](int kt, int m, uint4 (&v)[8]) {
        const bf16* p = b_ptr[m] + (size_t)kt * kKS * N;
#pragma unroll
        for (int r = 0; r < 8; ++r) v[r] = load_stream(p + (size_t)r * N);
    };
    auto mma = [&](const uint4 (&a)[MF], int m, const uint4 (&v)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const bf16x8 bf = block_column(v, c);
#pragma unroll
            for (int f = 0; f < MF; ++f)
                acc[f][m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, a[f]), bf, acc[f][m][c], 0, 0, 0);
        }
    };

    if (k0 < k1) {
        if constexpr (DUAL && MF == kMaxFrags) {
            // w1 of step kt+1 is loaded while the w3 half of step kt
            // computes, w3 of step kt+1 while the w1 half of step kt+1 does.
            // One step per iteration and the last step peeled, so every load
            // in the loop is unconditional: with 4 fragments' accumulators
            // (all 256 AGPRs) the register allocation of the two-step form
            // below spills.
            uint4 a[MF], v1[8], v3[8];
            load_a(k0, a);
            load_b(k0, 0, v1);
            load_b(k0, 1, v3);
            for (int kt = k0; kt + 1 < k1; ++kt) {
                mma(a, 0, v1);
                load_b(kt + 1, 0, v1);
                mma(a, 1, v3);
                load_a(kt + 1, a);
                load_b(kt + 1, 1, v3);
            }
            mma(a, 0, v1);
            mma(a, 1, v3);
        } else if constexpr (DUAL) {
            // The same staggered order, two steps per iteration (A rows of
            // the next step fetched ahead of its w1 block): 2% faster than
            // the one-step loop at 1 and 2 fragments.
            uint4 a0[MF], a1[MF], v1[8], v3[8];
            int kt = k0;
            load_a(kt, a0);
            load_b(kt, 0, v1);
            load_b(kt, 1, v3);
            for (; kt + 1 < k1; kt += 2) {
                mma(a0, 0, v1);
                load_a(kt + 1, a1);
                load_b(kt + 1, 0, v1);
                mma(a0, 1, v3);
                load_b(kt + 1, 1, v3);
                mma(a1, 0, v1);
                if (kt + 2 < k1) {
                    load_a(kt + 2, a0);
                    load_b(kt + 2, 0, v1);
                }
                mma(a1, 1, v3);
                if (kt + 2 < k1) load_b(kt + 2, 1, v3);
            }
            if (kt < k1) {
                mma(a0, 0, v1);
                mma(a0, 1, v3);
            }
        } else {
            // two steps of w2 in registers: step kt+1 loads while step kt
            // computes
            uint4 a0[MF], a1[MF], v0[8], v1[8];
            int kt = k0;
            load_a(kt, a0);
            load_b(kt, 0, v0);
            for (; kt + 1 < k1; kt += 2) {
                load_a(kt + 1, a1);
                load_b(kt + 1, 0, v1);
                mma(a0, 0, v0);
                if (kt + 2 < k1) {
                    load_a(kt + 2, a0);
                    load_b(kt + 2, 0, v0);
                }
                mma(a1, 0, v1);
            }
            if (kt < k1) mma(a0, 0, v0);
        }
    }

    if (KW > 1) {
        // ---- add the parts of K: the slab's first wave adds the others'
        // partial sums in K order; LDS slot of wave w (part p > 0):
        // (w / KW) (KW - 1) + p - 1
        if (kpart > 0) {
            const int slot = slab * (KW - 1) + kpart - 1;
#pragma unroll
            for (int f = 0; f < MF; ++f)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        red[slot * MF * NMAT * 8 + (f * NMAT + m) * 8 + c][lane] = acc[f][m][c];
        }
        __syncthreads();
        if (kpart != 0) return;
#pragma unroll
        for (int w = 0; w < KW - 1; ++w)
#pragma unroll
            for (int f = 0; f < MF; ++f)
#pragma unroll
                for (int m = 0; m < NMAT; ++m)
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        acc[f][m][c] += red[(slab * (KW - 1) + w) * MF * NMAT * 8 + (f * NMAT + m) * 8 + c][lane];
    }

    if (!b_ok) return;
#pragma unroll
    for (int f = 0; f < MF; ++f)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + kFrag * f + 4 * g + i;
            if (row >= row_end) continue;
            if (DUAL) {
                uint32_t w[4];
#pragma unroll
                for (int c2 = 0; c2 < 4; ++c2) {
                    const float h0 = silu_f32(acc[f][0][2 * c2][i]) * acc[f][1][2 * c2][i];
                    const float h1 = silu_f32(acc[f][0][2 * c2 + 1][i]) * acc[f][1][2 * c2 + 1][i];
                    w[c2] = pack_bf16x2(h0, h1);
                }
                *reinterpret_cast<uint4*>(reinterpret_cast<bf16*>(C) + (size_t)row * N + col) =
                    make_uint4(w[0], w[1], w[2], w[3]);
            } else {
                float* y = reinterpret_cast<float*>(C) + (size_t)split * R * N + (size_t)row * N + col;
                reinterpret_cast<float4*>(y)[0] =
                    make_float4(acc[f][0][0][i], acc[f][0][1][i], acc[f][0][2][i], acc[f][0][3][i]);
                reinterpret_cast<float4*>(y)[1] =
                    make_float4(acc[f][0][4][i], acc[f][0][5][i], acc[f][0][6][i], acc[f][0][7][i]);
            }
        }
}

// Row tiles: with KW > 1 tiles hold 16 rows (MF = 1); otherwise up to 64,
// with MF = 1, 2 or 4 by the tile's row count.
template <int KW>
constexpr int tile_rows() { return KW > 1 ? kFrag : kFrag * kMaxFrags; }

template <bool DUAL, int KW>
__global__ __launch_bounds__(kThreads) void stream_gemm_kernel(
    const bf16* __restrict__ A, const int32_t* __restrict__ a_rows, const bf16* __restrict__ B0,
    const bf16* __restrict__ B1, void* __restrict__ C, const int32_t* __restrict__ offsets, int R,
    int E, int K, int N, int splits) {
    constexpr int NMAT = DUAL ? 2 : 1;
    constexpr int TILE_N = (4 / KW) * kSlab;
    constexpr int TILE_M = tile_rows<KW>();
    // partial sums of the waves past the first of each slab (MF = 1)
    __shared__ floatx4 red[KW > 1 ? (4 - 4 / KW) * NMAT * 8 : 1][64];

    // ---- which (expert, split, n-tile, m-tile) this workgroup computes
    const int NT = (N + TILE_N - 1) / TILE_N;
    int total = 0;
    for (int e = 0; e < E; ++e) {
        const int n_e = offsets[e + 1] - offsets[e];
        total += ((n_e + TILE_M - 1) / TILE_M) * NT * splits;
    }
    const int per_xcd = (total + 7) / 8;
    const int slot = blockIdx.x >> 3;
    if (slot >= per_xcd) return;
    int L = (blockIdx.x & 7) * per_xcd + slot;
    if (L >= total) return;
    int e = 0, row0 = 0, row_end = 0, n_tile = 0, split = 0;
    for (e = 0; e < E; ++e) {
        const int o0 = offsets[e];
        const int n_e = offsets[e + 1] - o0;
        const int mt = (n_e + TILE_M - 1) / TILE_M;
        const int tiles = mt * NT * splits;
        if (L < tiles) {
            const int m = L % mt;
            const int rest = L / mt;
            n_tile = rest % NT;
            split = rest / NT;
            row0 = o0 + m * TILE_M;
            row_end = o0 + n_e;
            break;
        }
        L -= tiles;
    }

    const int KT = K / kKS;
    const int kt_split = (KT + splits - 1) / splits;
    const int s0 = min(split * kt_split, KT);
    const int s1 = min(s0 + kt_split, KT);
    const size_t b_base = (size_t)e * K * N;
    if constexpr (KW > 1) {
        stream_tile<DUAL, KW, 1>(A, a_rows, B0, B1, C, b_base, row0, row_end, n_tile, split, s0,
                                 s1, R, K, N, red);
    } else {
        const int rows = min(row_end - row0, TILE_M);
        if (rows <= kFrag)
            stream_tile<DUAL, 1, 1>(A, a_rows, B0, B1, C, b_base, row0, row_end, n_tile, split,
                                    s0, s1, R, K, N, red);
        else if (rows <= 2 * kFrag)
            stream_tile<DUAL, 1, 2>(A, a_rows, B0, B1, C, b_base, row0, row_end, n_tile, split,
                                    s0, s1, R, K, N, red);
        else
            stream_tile<DUAL, 1, 4>(A, a_rows, B0, B1, C, b_base, row0, row_end, n_tile, split,
                                    s0, s1, R, K, N, red);
    }
}

template <bool DUAL, int KW>
hipError_t launch_stream(const void* A, const int32_t* a_rows, const void* B0, const void* B1,
                         void* C, const int32_t* offsets, int R, int E, int K, int N, int splits,
                         hipStream_t stream) {
    const long long tile_n = (4 / KW) * kSlab;
    const long long NT = (N + tile_n - 1) / tile_n;
    const long long tile_m = tile_rows<KW>();
    const long long mtiles = (R + tile_m - 1) / tile_m + E;  // bound on sum_e ceil(n_e / tile_m)
    long long grid = mtiles * NT * splits;
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL((stream_gemm_kernel<DUAL, KW>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, reinterpret_cast<const bf16*>(A), a_rows,
                       reinterpret_cast<const bf16*>(B0), reinterpret_cast<const bf16*>(B1), C,
                       offsets, R, E, K, N, splits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm1_swiglu_stream(const void* x, const int32_t* row_token, const void* w1,
                                      const void* w3, const int32_t* offsets, int R, int E, int d,
                                      int f, int k_waves, void* h, hipStream_t stream) {
    if (k_waves == 4)
        return launch_stream<true, 4>(x, row_token, w1, w3, h, offsets, R, E, d, f, 1, stream);
    if (k_waves == 2)
        return launch_stream<true, 2>(x, row_token, w1, w3, h, offsets, R, E, d, f, 1, stream);
    return launch_stream<true, 1>(x, row_token, w1, w3, h, offsets, R, E, d, f, 1, stream);
}

hipError_t launch_gemm2_stream(const void* h, const void* w2, const int32_t* offsets, int R, int E,
                               int f, int d, int splits, float* y, hipStream_t stream) {
    return launch_stream<false, 1>(h, nullptr, w2, nullptr, y, offsets, R, E, f, d, splits,
                                       stream);
}

}  // namespace moe
