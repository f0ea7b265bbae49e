// gemm_bf16.hip -- the two expert contractions as grouped GEMMs on bf16 MFMA.
//
// Mixtral of Experts (wikillm.com card, "Method", SwiGLU pseudocode): each
// expert is w2 . (SiLU(w1 . x) * (w3 . x)).  With the rows of every expert
// grouped contiguously (route_permute.hip), the batch becomes, per expert e
// with rows [offsets[e], offsets[e+1]):
//   GEMM 1:  h = SiLU(X_e . w1[e]) * (X_e . w3[e])      X_e [n_e,d], w1/w3 [d,f]
//   GEMM 2:  y = h_e . w2[e]                            h_e [n_e,f], w2 [f,d]
// Both run as one launch over all experts.  The per-expert row counts stay on
// the device: the host sizes the grid for the worst case and each workgroup
// looks up its (expert, split, n-tile, m-tile) from offsets[]; surplus
// workgroups exit at once.
//
// Tile shape.  256 threads (4 wavefronts), K step 64, 256 weight columns
// staged per step (GEMM 1: 128 columns of w1 and the same 128 of w3; GEMM 2:
// 256 columns of w2).  BM rows per tile: 128 (waves 2x2) when experts have many
// rows, 32 (waves 1x4) when they have few.  The MFMA is
// v_mfma_f32_16x16x32_bf16: each lane feeds 8 consecutive k of one row (A) and
// of one column (B) and gets 4 fp32 results of one column.
//
// Operand staging.  X rows are K-contiguous: 16-byte global loads go to LDS as
// they are, each row's eight 16-byte chunks XOR-swizzled by (row/2)%8 so the
// fragment reads of 16 consecutive rows hit 16 distinct bank groups.  Weights
// are stored [k][n] (n contiguous), but a B fragment needs 8 consecutive k of
// one column, so each thread loads an 8x8 (k x n) block with eight 16-byte
// row loads, transposes it in registers with byte permutes, and writes eight
// 16-byte column pieces into 8 k-planes of LDS ([plane][column][8 k]), with
// column slots XOR-swizzled by (n/16)%8 so both the writes and the fragment
// reads are free of bank conflicts.
//
// Pipelining.  One LDS stage; the next K step's global loads are issued into
// registers before the current step's MFMAs, and written to LDS after a
// barrier.
//
// Tile order.  Workgroup IDs are dealt round-robin to the 8 XCDs, so the
// logical tile is (xcd * per_xcd + id / 8): each XCD walks a contiguous run of
// tiles, m-tile fastest, so the workgroups sharing a weight panel run together
// on one XCD and share its L2.
//
// Epilogues.  GEMM 1 applies SiLU(a) * b to the w1 / w3 accumulator pair of
// each element and stores h in bf16.  GEMM 2 stores fp32 y; with splits > 1
// the contraction is cut into equal K slices, each written to its own partial
// buffer (summed later in a fixed order, so results do not depend on timing).
#include "common.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 64;
constexpr int kLdsCols = 256;
constexpr int kPlanes = kBK / 8;

template <int BM, int WAVES_M, bool DUAL>
struct Cfg {
    static constexpr int WAVES_N = 4 / WAVES_M;
    static constexpr int BN = DUAL ? 128 : 256;  // output columns per tile
    static constexpr int WM = BM / WAVES_M;      // rows per wave
    static constexpr int FM = WM / 16;           // 16-row fragments per wave
    static constexpr int CW = BN / WAVES_N;      // output columns per wave
    static constexpr int FNH = CW / 16;          // 16-col fragments per wave per matrix
    static constexpr int FN = DUAL ? 2 * FNH : FNH;
    static constexpr int A_CHUNKS = BM * (kBK / 8) / kThreads;
    static_assert(WAVES_M * WAVES_N == 4, "4 waves");
    static_assert(FM >= 1 && WM % 16 == 0, "wave rows");
    static_assert(A_CHUNKS >= 1 && BM * (kBK / 8) % kThreads == 0, "A chunks");
};

__device__ __forceinline__ int a_slot(int row, int chunk) { return chunk ^ ((row >> 1) & 7); }
__device__ __forceinline__ int b_slot(int n) { return n ^ ((n >> 4) & 7); }

__device__ __forceinline__ uint32_t dw(const uint4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Column c (0..7) of an 8x8 bf16 block held as 8 row vectors: the 8 k values
// of that column, packed low k first.
__device__ __forceinline__ uint4 block_column(const uint4 (&v)[8], int c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    const int q = c >> 1;
    uint4 o;
    o.x = __builtin_amdgcn_perm(dw(v[1], q), dw(v[0], q), sel);
    o.y = __builtin_amdgcn_perm(dw(v[3], q), dw(v[2], q), sel);
    o.z = __builtin_amdgcn_perm(dw(v[5], q), dw(v[4], q), sel);
    o.w = __builtin_amdgcn_perm(dw(v[7], q), dw(v[6], q), sel);
    return o;
}

struct TileInfo {
    int valid;
    int e, split, n_tile, row0, row_end;
};

// Logical tile of this workgroup, or valid = 0.
template <int BM>
__device__ __forceinline__ TileInfo find_tile(const int32_t* __restrict__ offsets, int E, int NT,
                                              int splits) {
    TileInfo ti;
    ti.valid = 0;
    int total = 0;
    for (int e = 0; e < E; ++e) {
        const int n_e = offsets[e + 1] - offsets[e];
        total += ((n_e + BM - 1) / BM) * NT * splits;
    }
    const int per_xcd = (total + 7) / 8;
    const int slot = blockIdx.x >> 3;
    if (slot >= per_xcd) return ti;
    int L = (blockIdx.x & 7) * per_xcd + slot;
    if (L >= total) return ti;
    for (int e = 0; e < E; ++e) {
        const int o0 = offsets[e];
        const int n_e = offsets[e + 1] - o0;
        const int mt = (n_e + BM - 1) / BM;
        const int tiles = mt * NT * splits;
        if (L < tiles) {
            const int m = L % mt;
            const int rest = L / mt;
            ti.n_tile = rest % NT;
            ti.split = rest / NT;
            ti.e = e;
            ti.row0 = o0 + m * BM;
            ti.row_end = o0 + n_e;
            ti.valid = 1;
            return ti;
        }
        L -= tiles;
    }
    return ti;
}

template <int BM, int WAVES_M, bool DUAL>
__global__ __launch_bounds__(kThreads) void grouped_gemm_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B0, const bf16* __restrict__ B1,
    void* __restrict__ C, const int32_t* __restrict__ offsets, int R, int E, int K, int N,
    int splits) {
    using G = Cfg<BM, WAVES_M, DUAL>;
    __shared__ __align__(16) bf16 As[BM * kBK];
    __shared__ __align__(16) bf16 Bs[kPlanes * kLdsCols * 8];

    const int NT = (N + G::BN - 1) / G::BN;
    const TileInfo ti = find_tile<BM>(offsets, E, NT, splits);
    if (!ti.valid) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / G::WAVES_N;
    const int wn = wave % G::WAVES_N;
    const int col0 = ti.n_tile * G::BN;

    const int KT = K / kBK;
    const int kt_per = (KT + splits - 1) / splits;
    const int kt0 = min(ti.split * kt_per, KT);
    const int kt1 = min(kt0 + kt_per, KT);

    // ---- per-thread global load assignment
    // A: chunks tid + 256*i of the BM x 64 tile (8 chunks of 16 B per row).
    const bf16* a_src[G::A_CHUNKS];
    int a_lds[G::A_CHUNKS];
#pragma unroll
    for (int i = 0; i < G::A_CHUNKS; ++i) {
        const int chunk = tid + kThreads * i;
        const int row = chunk >> 3;
        const int c = chunk & 7;
        const int grow = min(ti.row0 + row, ti.row_end - 1);
        a_src[i] = A + (size_t)grow * K + c * 8;
        a_lds[i] = row * kBK + a_slot(row, c) * 8;
    }
    // B: one 8x8 (k x n) block per thread.
    int nb, kb, lds_col;
    const bf16* bmat;
    if (DUAL) {
        const int mat = tid >> 7;
        nb = tid & 15;
        kb = (tid >> 4) & 7;
        bmat = mat ? B1 : B0;
        lds_col = mat * 128 + nb * 8;
    } else {
        nb = tid & 31;
        kb = tid >> 5;
        bmat = B0;
        lds_col = nb * 8;
    }
    const int gcol = col0 + nb * 8;
    const bool b_ok = gcol < N;
    const bf16* b_src = bmat + (size_t)ti.e * K * N + (size_t)(kb * 8) * N + (b_ok ? gcol : 0);

    uint4 ra[G::A_CHUNKS];
    uint4 rb[8];

    auto load_global = [&](int kt) {
        // Unconditional loads: out-of-range rows and columns read clamped,
        // valid addresses and only feed outputs that are never stored.
#pragma unroll
        for (int i = 0; i < G::A_CHUNKS; ++i)
            ra[i] = *reinterpret_cast<const uint4*>(a_src[i] + (size_t)kt * kBK);
        const bf16* p = b_src + (size_t)kt * kBK * N;
#pragma unroll
        for (int r = 0; r < 8; ++r) rb[r] = *reinterpret_cast<const uint4*>(p + (size_t)r * N);
    };
    auto store_lds = [&]() {
#pragma unroll
        for (int i = 0; i < G::A_CHUNKS; ++i) *reinterpret_cast<uint4*>(As + a_lds[i]) = ra[i];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int n = lds_col + c;
            *reinterpret_cast<uint4*>(Bs + kb * (kLdsCols * 8) + b_slot(n) * 8) =
                block_column(rb, c);
        }
    };

    floatx4 acc[G::FM][G::FN];
#pragma unroll
    for (int m = 0; m < G::FM; ++m)
#pragma unroll
        for (int f = 0; f < G::FN; ++f) acc[m][f] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Fragment addressing (elements) that does not change with the K step.
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;
    int a_frag_row[G::FM];
#pragma unroll
    for (int m = 0; m < G::FM; ++m) a_frag_row[m] = wm * G::WM + 16 * m + lrow;
    int b_frag_slot[G::FN];
#pragma unroll
    for (int f = 0; f < G::FN; ++f) {
        int base;
        if (DUAL) base = (f < G::FNH) ? wn * G::CW + 16 * f : 128 + wn * G::CW + 16 * (f - G::FNH);
        else base = wn * G::CW + 16 * f;
        b_frag_slot[f] = b_slot(base + lrow) * 8;
    }

    if (kt0 < kt1) {
        load_global(kt0);
        store_lds();
        __syncthreads();
    }
    for (int kt = kt0; kt < kt1; ++kt) {
        const bool more = kt + 1 < kt1;
        if (more) load_global(kt + 1);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int chunk = 4 * s + lgrp;
            bf16x8 af[G::FM];
#pragma unroll
            for (int m = 0; m < G::FM; ++m) {
                const int row = a_frag_row[m];
                af[m] = *reinterpret_cast<const bf16x8*>(As + row * kBK + a_slot(row, chunk) * 8);
            }
            const bf16* bplane = Bs + chunk * (kLdsCols * 8);
#pragma unroll
            for (int f = 0; f < G::FN; ++f) {
                const bf16x8 bf = *reinterpret_cast<const bf16x8*>(bplane + b_frag_slot[f]);
#pragma unroll
                for (int m = 0; m < G::FM; ++m)
                    acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bf, acc[m][f], 0, 0, 0);
            }
        }
        if (more) {
            __syncthreads();
            store_lds();
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds rows 4*lgrp + i (i = 0..3) of column lrow of
    // each 16x16 fragment.
#pragma unroll
    for (int m = 0; m < G::FM; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int grow = ti.row0 + wm * G::WM + 16 * m + 4 * lgrp + i;
            if (grow >= ti.row_end) continue;
            if (DUAL) {
                bf16* h = reinterpret_cast<bf16*>(C);
#pragma unroll
                for (int f = 0; f < G::FNH; ++f) {
                    const int col = col0 + wn * G::CW + 16 * f + lrow;
                    if (col < N) {
                        const float a = acc[m][f][i];
                        const float b = acc[m][f + G::FNH][i];
                        const float hv = silu_f32(a) * b;
                        reinterpret_cast<uint16_t*>(h)[(size_t)grow * N + col] =
                            (uint16_t)f32_to_bf16_bits(hv);
                    }
                }
            } else {
                float* y = reinterpret_cast<float*>(C) + (size_t)ti.split * R * N;
#pragma unroll
                for (int f = 0; f < G::FN; ++f) {
                    const int col = col0 + wn * G::CW + 16 * f + lrow;
                    if (col < N) y[(size_t)grow * N + col] = acc[m][f][i];
                }
            }
        }
    }
}

template <int BM, int WAVES_M, bool DUAL>
hipError_t launch_grouped(const void* A, const void* B0, const void* B1, void* C,
                          const int32_t* offsets, int R, int E, int K, int N, int splits,
                          hipStream_t stream) {
    using G = Cfg<BM, WAVES_M, DUAL>;
    const int NT = (N + G::BN - 1) / G::BN;
    const long long mtiles = (R + BM - 1) / BM + E;  // bound on sum_e ceil(n_e / BM)
    long long grid = mtiles * NT * splits;
    grid = (grid + 7) / 8 * 8;
    hipLaunchKernelGGL((grouped_gemm_kernel<BM, WAVES_M, DUAL>), dim3((unsigned)grid),
                       dim3(kThreads), 0, stream, reinterpret_cast<const bf16*>(A),
                       reinterpret_cast<const bf16*>(B0), reinterpret_cast<const bf16*>(B1), C,
                       offsets, R, E, K, N, splits);
    return hipGetLastError();
}

}  // namespace

int gemm_bm(int variant) { return variant == GEMM_SMALL_M ? 32 : 128; }
int gemm1_bn(int) { return 128; }
int gemm2_bn(int) { return 256; }

hipError_t launch_gemm1_swiglu_bf16(int variant, const void* x_perm, const void* w1,
                                    const void* w3, const int32_t* offsets, int R, int E, int d,
                                    int f, void* h, hipStream_t stream) {
    if (variant == GEMM_SMALL_M)
        return launch_grouped<32, 1, true>(x_perm, w1, w3, h, offsets, R, E, d, f, 1, stream);
    return launch_grouped<128, 2, true>(x_perm, w1, w3, h, offsets, R, E, d, f, 1, stream);
}

hipError_t launch_gemm2_bf16(int variant, const void* h, const void* w2, const int32_t* offsets,
                             int R, int E, int f, int d, int splits, float* y,
                             hipStream_t stream) {
    if (variant == GEMM_SMALL_M)
        return launch_grouped<32, 1, false>(h, w2, nullptr, y, offsets, R, E, f, d, splits, stream);
    return launch_grouped<128, 2, false>(h, w2, nullptr, y, offsets, R, E, f, d, splits, stream);
}

}  // namespace moe
