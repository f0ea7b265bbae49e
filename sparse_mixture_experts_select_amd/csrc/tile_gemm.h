// tile_gemm.h -- the expert contractions for batches with many rows per
// expert (prefill), where the time is MFMA work: 256x256 macro tiles.  The
// kernels and their launch; gemm_tile.hip and gemm_tile_nt.hip instantiate
// them (see NT_B below).
//
// Same products as the other GEMM files (Mixtral of Experts, wikillm.com card,
// "Method", SwiGLU pseudocode): per expert e over its grouped rows,
//   GEMM 1:  h = SiLU(X_e . w1[e]) * (X_e . w3[e])
//   GEMM 2:  y = h_e . w2[e]   (fp32)
//
// Workgroup: 256 threads = 4 wavefronts in a 2x2 grid.  Macro tile: 256 rows x
// 256 weight columns (GEMM 1: 128 columns of w1 and the same 128 of w3; GEMM 2:
// 256 columns of w2), K step 32.  Each wave owns 128 rows x 128 columns of
// accumulators (8 x 8 fragments of v_mfma_f32_16x16x32_bf16, 256 fp32 per
// lane, held in AGPRs), so every fragment read from LDS feeds 8 MFMAs; its
// rows are the tile's alternate 16-row fragments (wave row wm: fragments
// wm, wm + 2, ...), so that in a tile with fewer than 256 rows both wave rows
// can skip their empty fragments alike.
//
// Tail tiles.  An expert's rows past its last multiple of 256, when there are
// at most 128 of them, form a tail tile of 128 rows x two column tiles: the
// two row halves of the waves (wm) take one column tile each, all waves read
// the same 128 A rows.  Such a tile loads 8 KiB of A and 32 KiB of B per K
// step (40 KiB against 32 KiB for a full tile) and covers two column tiles,
// where a 256-row tile would spend a full tile's loads and MFMAs per column
// tile on rows that do not exist.  The kernel is data-movement bound, so a
// tail tile costs about 1.25 full tiles for the work of two.  Its waves all
// hold the same rows, so a tail tile multiplies only the 16-row fragments
// that hold some of them (2 up to 32 rows, 4 up to 64, 6 up to 96, else all
// 8), and a full tile with at most 192 rows 6 per wave: each fragment count
// is its own expansion of the K loop, chosen per tile.
//
// Staging: global -> LDS by DMA (buffer_load_dwordx4 ... lds: lane l's 16
// bytes land at the wave's LDS base + 16 l).  SGPR buffer descriptors over A
// and the expert's weights; each lane's byte offset is fixed for the whole
// loop and a wave-uniform offset advances per K step.  Four LDS stages of
// 40 KiB (a full tile uses 32 KiB of each), loads three K steps ahead.  The
// one barrier of a step sits half way through its MFMAs: before it each wave waits for its own loads of the
// next stage (always exactly vmcnt(8), vmcnt(10) in a tail tile: past the
// end the refills repeat the last step, valid addresses never read); after it the wave refills the
// stage of the previous step and reads the next step's A fragments under the
// second half of the MFMAs, so a step starts with its operands in registers.
// No register holds staged data and no VALU work is spent on it.  The
// barrier is a raw s_barrier between compiler-only fences, so loads of later
// steps stay in flight across it.  Each stage is its own LDS array and the K
// loop is unrolled by four, so every read and every refill names a fixed
// array, and the compiler's own waits for the DMA stay per stage.

// LDS layouts (both bank-conflict free for the fragment reads):
//   A stage: [256 rows][32 k], 64 bytes per row; the row's four 16-byte
//     chunks are stored XOR (row/2)%4.  A fragment read (ds_read_b128, one
//     16-byte chunk per lane, 16 rows) then spreads over all 64 banks; the
//     plain row order, or an XOR with (row/4)%4, leaves it 2-way conflicted
//     (measured: half the read rate).
//   B stage: two halves of [32 k][128 n] (GEMM 1: w1 | w3; GEMM 2: columns
//     0..127 | 128..255), the weights' own orientation (n contiguous), 256
//     bytes per k row in 32-byte groups of 16 columns; group G of row k is
//     stored at G XOR ((k%4) | ((k/8)%2) << 2).  A B fragment (8 k x 16 n per
//     lane group) is read with two ds_read_b64_tr_b16, which hand each lane 4
//     consecutive k of one column from a 4 x 16 tile whose rows the 16 lanes
//     address in 8-byte pieces.
// The DMA lane order fixes the LDS address, so each lane simply loads the
// global chunk that belongs at its swizzled LDS position.
//
// Order.  Tiles are numbered by expert, then bands of 8 full row tiles (the
// last band of an expert also takes its tail row); within a band, pairs of
// column tiles in order, each pair's full-row tiles rows fastest, then its
// tail tile.  Each XCD takes a contiguous run of ceil(n/8) tile numbers
// (workgroup IDs are dealt to the 8 XCDs round-robin), so the workgroups
// that run together on an XCD share A rows and weight panels in one L2: an
// expert with many rows runs as rounds of 8 row tiles x 4 column tiles, and
// consecutive rounds of a band keep its 8 A slabs.
//
// Last round (GEMM 2).  An XCD's tiles run in rounds of its CUs; the tiles
// of its last, partial round may be cut into p equal K ranges (p chosen per
// XCD from a cost in K steps: rounds x (steps per piece + fill and epilogue)
// + the partial sums' traffic), so that round keeps more CUs busy while all
// workgroups still walk K in step.  A piece writes its fp32 accumulators to
// a partial-sum slot; tile_fixup_kernel then sums the pieces of each cut
// tile in piece order and stores y.  GEMM 1 tiles are never cut: with its
// SwiGLU epilogue the fixup cost more than the rounds saved (measured).
//
// Epilogue.  GEMM 1 forms SiLU(a) * b, stages the bf16 tile in LDS (two of the
// stage arrays, 16-byte chunks XOR-swizzled by row) and writes it with 16-byte
// row-contiguous stores.  GEMM 2 writes fp32 straight from the
// accumulators (64-byte row segments per fragment).
#pragma once

#include "common.h"
#include "tile_order.h"

#include <atomic>

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kBK = 32;
constexpr int kStageBytes = 40 * 1024;  // full tile: A 16 KiB + B 16 KiB; tail tile: A 8 + B 32
constexpr int kBOffFull = 16 * 1024;    // B part of a stage, full tile
constexpr int kBOffTail = 8 * 1024;     // B part of a stage, tail tile
constexpr int kBHalfBytes = kBK * 128 * 2;  // one 128-column block of B (8 KiB)

typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) short4_t lds_short4;

__device__ __forceinline__ int b_group_swz(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }

// vmcnt(n) with the other counters left alone (gfx9 s_waitcnt encoding).
#define MOE_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | 0x70 | 0xF00 | (((n) >> 4) << 14))

// Barrier inside each K step.  Every LDS read of the stage about to be
// refilled was consumed by an MFMA of the previous step (so it has completed
// and no count wait is needed here); the compiler-only fences keep memory
// accesses from moving across the barrier, and DMA loads of later steps stay
// in flight.
__device__ __forceinline__ void stage_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

constexpr int kSlotFloats = kThreads * 256;  // one tile's fp32 accumulators
// The partial-sum buffer starts with a header written by the tile kernel for
// the fixup: ints [8 x] = the number of cut tiles of XCD x, then from int 64
// one 8-int descriptor per cut tile {row0, row_end, col0, is_tail, first
// slot, pieces}, cut tiles numbered XCD by XCD.  The slots follow.
constexpr int kHeaderFloats = 64 + 8 * 8 * kMaxCpx;

// ---- GEMM 1 epilogue of one tile: lane holds rows 4*lgrp + r (r = 0..3) of
// column lrow of each fragment.  st0 and st1 are two LDS arrays of at least
// 32 KiB that h is staged through.
template <bool DUAL>
__device__ __forceinline__ void tile_epilogue(const floatx4 (&acc)[8][8], const TileGeo& geo,
                                              void* __restrict__ C, int R, int N, int kb,
                                              unsigned char* st0, unsigned char* st1) {
    constexpr int BN = DUAL ? 128 : 256;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;
    const int row0 = geo.row0, row_end = geo.row_end, col0 = geo.col0;
    const bool is_tail = geo.is_tail;
    if (DUAL) {
        __syncthreads();  // every wave is done reading the stages
        // Stage the wave pair's 128 x 128 bf16 block of h in LDS (wm = 0 in
        // st0, wm = 1 in st1; full tile: the wave row's alternate 16-row
        // fragments, block row rr = tile row 32 (rr/16) + 16 wm + rr%16; tail
        // tile: first | second column tile), 256 bytes per row, 16-byte chunk
        // ch of row r stored at ch ^ (r % 16).
        uint16_t* hs_w = reinterpret_cast<uint16_t*>(wm == 0 ? st0 : st1);
#pragma unroll
        for (int m = 0; m < 8; ++m)
#pragma unroll
            for (int n = 0; n < 4; ++n)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * m + 4 * lgrp + r;  // within the block's 128 rows
                    const int c = wn * 64 + 16 * n + lrow;
                    const float hv = silu_f32(acc[m][n][r]) * acc[m][n + 4][r];
                    hs_w[row * 128 + (((c >> 3) ^ (row & 15)) << 3) + (c & 7)] =
                        (uint16_t)f32_to_bf16_bits(hv);
                }
        __syncthreads();
        uint16_t* h = reinterpret_cast<uint16_t*>(C);
        // staged row sr = 0..255: block sr/128, row sr%128 of that block
        if (kb) {
            // K-blocked h: for each block of 32 columns, consecutive rows are
            // one contiguous run of 64-byte row pieces.
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int idx = tid + kThreads * q;
                const int piece = idx & 3;        // 16-byte piece of the 64-byte row segment
                const int sr = (idx >> 2) & 255;
                const int b = idx >> 10;          // block of 32 columns within the 128
                const int ch = 4 * b + piece;     // 16-byte chunk of the staged row
                const int rr = sr & 127;
                const int grow = row0 + (is_tail ? rr : 32 * (rr >> 4) + 16 * (sr >> 7) + (rr & 15));
                const int gc = col0 + (is_tail ? (sr >> 7) * BN : 0) + ch * 8;
                const uint16_t* hs_r = reinterpret_cast<const uint16_t*>(sr < 128 ? st0 : st1);
                if (grow < row_end && gc < N)
                    *reinterpret_cast<uint4*>(h + ((size_t)(gc >> 5) * R + grow) * 32 + (gc & 31)) =
                        *reinterpret_cast<const uint4*>(hs_r + rr * 128 + ((ch ^ (rr & 15)) << 3));
            }
        } else {
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int idx = tid + kThreads * q;
                const int sr = idx >> 4;    // 0..255
                const int ch = idx & 15;    // 16-byte chunk of the row
                const int rr = sr & 127;
                const int grow = row0 + (is_tail ? rr : 32 * (rr >> 4) + 16 * (sr >> 7) + (rr & 15));
                const int gc = col0 + (is_tail ? (sr >> 7) * BN : 0) + ch * 8;
                const uint16_t* hs_r = reinterpret_cast<const uint16_t*>(sr < 128 ? st0 : st1);
                if (grow < row_end && gc < N)
                    *reinterpret_cast<uint4*>(h + (size_t)grow * N + gc) =
                        *reinterpret_cast<const uint4*>(hs_r + rr * 128 + ((ch ^ (rr & 15)) << 3));
            }
        }
    }
}

// NT_B: the weight DMA marked nontemporal -- for launches whose weight
// panels are each read by one row tile (GEMM 2, and GEMM 1 at up to ~192
// rows per expert), where HBM then serves the stream faster; where several
// row tiles share a panel through L2 the hint costs GEMM 1 6-11%.
template <bool DUAL, bool NT_B>
__global__ __launch_bounds__(kThreads, 1) void tile_gemm_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ B0, const bf16* __restrict__ B1,
    void* __restrict__ C, float* __restrict__ partials, const int32_t* __restrict__ offsets, int R,
    int E, int K, int N, int cpx, int max_pieces, int kb) {
    constexpr int BN = DUAL ? 128 : 256;  // output columns per column tile
    // One array per stage: the compiler can then tell the stage being read
    // from the stages the DMA is writing, and does not wait for those loads.
    __shared__ __align__(16) unsigned char st0[kStageBytes];
    __shared__ __align__(16) unsigned char st1[kStageBytes];
    __shared__ __align__(16) unsigned char st2[kStageBytes];
    __shared__ __align__(16) unsigned char st3[kStageBytes];

    // ---- this workgroup's item: a whole tile, or one K piece of a tile
    const int NT = (N + BN - 1) / BN;
    const int NTP = (NT + 1) / 2;
    const int KT = K / kBK;
    const int n_tiles = count_tiles(offsets, E, NT, NTP);
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    if (DUAL) {
        // GEMM 1: whole tiles only (no schedule, no partial sums)
        const int per_xcd = (n_tiles + 7) / 8;
        if (slot >= per_xcd || xcd * per_xcd + slot >= n_tiles) return;
    }
    const XcdSched sc = DUAL ? XcdSched{xcd * ((n_tiles + 7) / 8), n_tiles, 0, 1}
                             : xcd_schedule(n_tiles, xcd, cpx, KT, max_pieces);
    if (!DUAL && slot == 0 && threadIdx.x == 0)
        reinterpret_cast<int*>(partials)[8 * xcd] = sc.p > 1 ? sc.r : 0;
    if (slot >= sc.full + sc.r * sc.p) return;
    int t, kt0 = 0, kt1 = KT, piece = -1, rt = 0;
    if (slot < sc.full) {
        t = sc.start + slot;
    } else {
        const int u = slot - sc.full;
        rt = u % sc.r;
        t = sc.start + sc.full + rt;
        if (sc.p > 1) {
            piece = u / sc.r;
            kt0 = piece * KT / sc.p;
            kt1 = (piece + 1) * KT / sc.p;
        }
    }
    const TileGeo geo = tile_geometry(t, offsets, E, NT, NTP, BN);
    const int e = geo.e, row0 = geo.row0, row_end = geo.row_end, col0 = geo.col0;
    const bool is_tail = geo.is_tail;
    // A K piece's partial-sum slot and cut-tile number, found here, where
    // they cost two wave-uniform scalars (after the K loop the search would
    // compete with the accumulators for registers).
    XcdBases piece_bases{0, 0};
    if (!DUAL && piece >= 0) piece_bases = xcd_bases(n_tiles, xcd, cpx, KT, max_pieces);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform, so the DMA loads' LDS destinations (M0) are formed in
    // scalar registers instead of being read back from a vector register
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1;
    const int wn = wave & 1;
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;


    // ---- DMA sources.  Buffer descriptors (SGPRs) over A and over the
    // expert's weight matrices; per lane a loop-invariant byte offset, per K
    // step a wave-uniform one.  Unit u = 256 i + 64 wave + lane of each stage
    // part; the wave's LDS destination for instruction i is part base +
    // (256 i + 64 wave) * 16.  A: 4 instructions (256 rows; 2 in a tail tile),
    // B: 4 (two 128-column blocks; 8 and four blocks in a tail tile).
    const __amdgpu_buffer_rsrc_t a_rsrc =
        __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, 0x7fffffff, 0x00020000);
    const bf16* bh0 = B0 + (size_t)e * K * N;
    const bf16* bh1 = (DUAL ? B1 : B0) + (size_t)e * K * N;
    const __amdgpu_buffer_rsrc_t b_rsrc0 =
        __builtin_amdgcn_make_buffer_rsrc((void*)bh0, (short)0, 0x7fffffff, 0x00020000);
    const __amdgpu_buffer_rsrc_t b_rsrc1 =
        __builtin_amdgcn_make_buffer_rsrc((void*)bh1, (short)0, 0x7fffffff, 0x00020000);
    int a_voff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int u = 256 * i + 64 * wave + lane;
        // row r = u/4; stored chunk u%4 holds logical chunk (u%4) ^ ((r/2)%4).
        const int r = u >> 2;
        const int c = (u & 3) ^ ((r >> 1) & 3);
        const int grow = min(row0 + r, row_end - 1);  // rows past the expert only feed unstored rows
        // row-major A: row grow at grow * K; K-blocked A: block kt at kt * R * 32,
        // row grow at grow * 32 within it (one K step of 256 rows is 16 KiB
        // of contiguous memory, read in full 128-byte lines)
        a_voff[i] = (kb ? grow * 32 + 8 * c : grow * K + 8 * c) * 2;
    }
    // B block h of the stage (h = i/2): GEMM 1 full tile: w1 | w3 of the
    // column tile; tail: w1 | w3 of the first column tile, then of the second.
    // GEMM 2: 128-column blocks left to right (one column tile per two
    // blocks).  Within a block, k row kk = (u%512)/16 and stored unit p = u%16
    // is group (p/2) ^ swz(kk), 8-column piece p%2.
    int b_voff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int u = 256 * i + 64 * wave + lane;
        const int v = u & 511;
        const int kk = v >> 4;
        const int p = v & 15;
        const int col = 16 * ((p >> 1) ^ b_group_swz(kk)) + 8 * (p & 1);
        const int h = i >> 1;
        int gcol = (DUAL ? col0 + BN * (h >> 1) : col0 + 128 * h) + col;
        if (gcol >= N) gcol = 0;  // columns past N only feed unstored columns
        b_voff[i] = (kk * N + gcol) * 2;
    }
    const int a_step = kb ? R * kBK * 2 : kBK * 2;  // bytes per K step in A
    const int b_step = kBK * N * 2;                 // bytes per K step in B

    // ---- fragment addressing (bytes within a stage)
    // A fragment m: in a full tile the tile's 16-row fragment 2 m + wm (the
    // two wave rows take alternate fragments, so a tile with fewer than 256
    // rows leaves both about equally empty), in a tail tile fragment m of the
    // tail's 128 rows for every wave; lane row lrow, chunk lgrp, stored at
    // chunk lgrp ^ ((row/2)%4) = lgrp ^ ((lrow/2)%4).  Fragment m + 1 lies
    // 32 rows (full) or 16 rows (tail) further on.
    const int a_frag = ((is_tail ? 0 : wm * 16) + lrow) * 64 + 16 * (lgrp ^ ((lrow >> 1) & 3));
    // B fragment n: 16 columns of one block; lane (lgrp, lrow) addresses k row
    // 8 lgrp + lrow/4 (+4 for the second read), columns 4 (lrow%4) .. +3.
    const int b_k = 8 * lgrp + (lrow >> 2);
    const int b_swz = b_group_swz(b_k);  // the same for b_k + 4
    int b_frag[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        int blk, g;
        if (DUAL) {
            blk = (is_tail ? 2 * wm : 0) + (n >> 2);
            g = 4 * wn + (n & 3);
        } else {
            blk = (is_tail ? 2 * wm : 0) + wn;
            g = n;
        }
        b_frag[n] = (is_tail ? kBOffTail : kBOffFull) + blk * kBHalfBytes + b_k * 256 +
                    32 * (g ^ b_swz) + 8 * (lrow & 3);
    }

    floatx4 acc[8][8];
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int n = 0; n < 8; ++n) acc[m][n] = floatx4{0.f, 0.f, 0.f, 0.f};

    // Loads of one K step: NA_ A and NB_ B instructions per lane.
#define MOE_ISSUE_STAGE(KT_, ARR_, NA_, NB_, BOFF_)                                         \
    do {                                                                                    \
        lds_char* sb_ = (lds_char*)(lds_void*)(ARR_) + (64 * wave) * 16;                    \
        const int ka_ = (KT_) * a_step;                                                     \
        const int kb_ = (KT_) * b_step;                                                     \
        _Pragma("unroll") for (int i_ = 0; i_ < (NA_); ++i_)                                \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(a_rsrc, (lds_void*)(sb_ + 4096 * i_), \
                                                     16, a_voff[i_], ka_, 0, 0);            \
        _Pragma("unroll") for (int i_ = 0; i_ < (NB_); ++i_)                                \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                       \
                (DUAL ? ((i_ >> 1) & 1) : 0) ? b_rsrc1 : b_rsrc0,                            \
                (lds_void*)(sb_ + (BOFF_) + 4096 * i_), 16, b_voff[i_], kb_, 0,             \
                NT_B ? 2 : 0);                                                              \
    } while (0)

#define MOE_READ_A(ARR_, M_)                                                                \
    (*reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>(                    \
        (const lds_char*)(lds_void*)(ARR_) + a_frag + (M_) * a_mstride_))

#define MOE_READ_B(ST_, N_)                                                                 \
    __builtin_bit_cast(bf16x8, __builtin_shufflevector(                                     \
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((ST_) + b_frag[N_])),        \
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)((ST_) + b_frag[N_] + 4 * 256)), \
        0, 1, 2, 3, 4, 5, 6, 7))

#define MOE_MFMAS(N_, BF_, MF_)                                                             \
    _Pragma("unroll") for (int m_ = 0; m_ < (MF_); ++m_)                                    \
        acc[m_][N_] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afc_[m_], BF_, acc[m_][N_], 0, 0, 0)

// Scheduling hints: within a group of 8 (or 6) MFMAs, put one of the group's
// LDS reads (for fragments two groups ahead) after each of the first NR_
// MFMAs, and NV_ of the stage refill's DMA loads among the later MFMAs, so
// the wave never holds a burst of memory instructions while the matrix core
// idles.  Loops of 2 or 4 fragments are left to the compiler.
#define MOE_SCHED_GROUP(NR_, NV_)                                                           \
    _Pragma("unroll") for (int i_ = 0; i_ < 8; ++i_) {                                      \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        if (i_ < (NR_)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                  \
        if ((i_ == 2 && (NV_) > 0) || (i_ == 5 && (NV_) > 1) || (i_ == 7 && (NV_) > 2))     \
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                              \
    }
#define MOE_SCHED_GROUP6(NR_, NV_)                                                          \
    _Pragma("unroll") for (int i_ = 0; i_ < 6; ++i_) {                                      \
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                                  \
        if (i_ < (NR_)) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                  \
        if ((i_ == 1 && (NV_) > 0) || (i_ == 4 && (NV_) > 1) || (i_ == 5 && (NV_) > 2))     \
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                              \
    }

    // One K step on stage CUR_.  On entry AF_ holds its A fragments and
    // bq0, bq1 its first two B fragments; B fragment n + 2 is read while the
    // MFMAs of fragment n run.  Half way (before fragment 4): wait until this
    // wave's loads of the next stage NXT_ are complete (vmcnt(NV_): only the
    // stage after it may still be in flight), barrier (now every wave's loads
    // of NXT_ have landed, and every wave has consumed its reads of REF_, the
    // stage of the previous step), refill REF_ with step kt + 3, and read the
    // next step's A fragments (into AN_) and first two B fragments from NXT_
    // under the remaining MFMAs.  The two A arrays trade roles from step to
    // step (the unroll by four names them), so no register copy moves the
    // fragments between steps.
    // A step past the end of the slice (the last loop iteration may hold up
    // to three) skips its reads and MFMAs but still waits, takes the barrier
    // and issues its (repeated, never read) refill, so every path through the
    // loop issues the same sequence of DMA loads: the compiler's DMA wait
    // tracking then stays per stage across the guards' control-flow merges.
#define MOE_STEP(CUR_, NXT_, REF_, AF_, AN_, NA_, NB_, BOFF_, MF_, G4_, G5_, G6_, G7_)    \
    {                                                                                       \
        const lds_char* st_ = (const lds_char*)(lds_void*)(CUR_);                           \
        bf16x8(&afc_)[8] = (AF_);                                                           \
        const bool live_ = kt < kt1;                                                        \
        bf16x8 b4_, b5_;                                                                    \
        if (live_) {                                                                        \
            const bf16x8 b2_ = MOE_READ_B(st_, 2);                                          \
            MOE_MFMAS(0, bq0, MF_);                                                         \
            const bf16x8 b3_ = MOE_READ_B(st_, 3);                                          \
            MOE_MFMAS(1, bq1, MF_);                                                         \
            b4_ = MOE_READ_B(st_, 4);                                                       \
            MOE_MFMAS(2, b2_, MF_);                                                         \
            b5_ = MOE_READ_B(st_, 5);                                                       \
            MOE_MFMAS(3, b3_, MF_);                                                         \
            if constexpr ((MF_) == 8) {                                                     \
                MOE_SCHED_GROUP(2, 0);                                                      \
                MOE_SCHED_GROUP(2, 0);                                                      \
                MOE_SCHED_GROUP(2, 0);                                                      \
                MOE_SCHED_GROUP(2, 0);                                                      \
            } else if constexpr ((MF_) == 6) {                                              \
                MOE_SCHED_GROUP6(2, 0);                                                     \
                MOE_SCHED_GROUP6(2, 0);                                                     \
                MOE_SCHED_GROUP6(2, 0);                                                     \
                MOE_SCHED_GROUP6(2, 0);                                                     \
            }                                                                               \
        }                                                                                   \
        MOE_WAIT_VM((NA_) + (NB_));                                                         \
        stage_barrier();                                                                    \
        MOE_ISSUE_STAGE(min(kt + 3, kt1 - 1), REF_, NA_, NB_, BOFF_);                       \
        if (live_) {                                                                        \
            const lds_char* sn_ = (const lds_char*)(lds_void*)(NXT_);                       \
            const bf16x8 b6_ = MOE_READ_B(st_, 6);                                          \
            if constexpr (0 < (MF_)) AN_[0] = MOE_READ_A(NXT_, 0);                           \
            if constexpr (1 < (MF_)) AN_[1] = MOE_READ_A(NXT_, 1);                           \
            MOE_MFMAS(4, b4_, MF_);                                                         \
            const bf16x8 b7_ = MOE_READ_B(st_, 7);                                          \
            if constexpr (2 < (MF_)) AN_[2] = MOE_READ_A(NXT_, 2);                           \
            if constexpr (3 < (MF_)) AN_[3] = MOE_READ_A(NXT_, 3);                           \
            MOE_MFMAS(5, b5_, MF_);                                                         \
            if constexpr (4 < (MF_)) AN_[4] = MOE_READ_A(NXT_, 4);                           \
            if constexpr (5 < (MF_)) AN_[5] = MOE_READ_A(NXT_, 5);                           \
            if constexpr (6 < (MF_)) AN_[6] = MOE_READ_A(NXT_, 6);                           \
            if constexpr (7 < (MF_)) AN_[7] = MOE_READ_A(NXT_, 7);                           \
            bq0 = MOE_READ_B(sn_, 0);                                                       \
            MOE_MFMAS(6, b6_, MF_);                                                         \
            bq1 = MOE_READ_B(sn_, 1);                                                       \
            MOE_MFMAS(7, b7_, MF_);                                                         \
            if constexpr ((MF_) == 8) {                                                     \
                MOE_SCHED_GROUP(4, G4_);                                                    \
                MOE_SCHED_GROUP(4, G5_);                                                    \
                MOE_SCHED_GROUP(6, G6_);                                                    \
                MOE_SCHED_GROUP(2, G7_);                                                    \
            } else if constexpr ((MF_) == 6) {                                              \
                MOE_SCHED_GROUP6(4, G4_);                                                   \
                MOE_SCHED_GROUP6(4, G5_);                                                   \
                MOE_SCHED_GROUP6(4, G6_);                                                   \
                MOE_SCHED_GROUP6(2, G7_);                                                   \
            }                                                                               \
        }                                                                                   \
        ++kt;                                                                               \
    }

    // The K loop for one tile shape.  Loads in flight: the prologue fills
    // st0, st1, st2 with steps kt0, kt0+1, kt0+2 and waits for the first;
    // each step refills one stage half way through, so at every half-way wait
    // exactly two younger steps are in flight and one fixed vmcnt leaves the
    // next step's loads complete.  Past the last step the refills repeat it
    // (valid addresses, never read).
#define MOE_K_LOOP(NA_, NB_, BOFF_, MF_, AMS_, G4_, G5_, G6_, G7_)                          \
    {                                                                                       \
        constexpr int a_mstride_ = (AMS_);                                                  \
        MOE_ISSUE_STAGE(kt0, st0, NA_, NB_, BOFF_);                                         \
        MOE_ISSUE_STAGE(min(kt0 + 1, kt1 - 1), st1, NA_, NB_, BOFF_);                       \
        MOE_ISSUE_STAGE(min(kt0 + 2, kt1 - 1), st2, NA_, NB_, BOFF_);                       \
        MOE_WAIT_VM(2 * ((NA_) + (NB_)));                                                   \
        stage_barrier();                                                                    \
        bf16x8 af0[8], af1[8];                                                              \
        _Pragma("unroll") for (int m = 0; m < (MF_); ++m) af0[m] = MOE_READ_A(st0, m);      \
        const lds_char* s0_ = (const lds_char*)(lds_void*)st0;                              \
        bf16x8 bq0 = MOE_READ_B(s0_, 0);                                                    \
        bf16x8 bq1 = MOE_READ_B(s0_, 1);                                                    \
        while (kt < kt1) {                                                                  \
            MOE_STEP(st0, st1, st3, af0, af1, NA_, NB_, BOFF_, MF_, G4_, G5_, G6_, G7_)     \
            MOE_STEP(st1, st2, st0, af1, af0, NA_, NB_, BOFF_, MF_, G4_, G5_, G6_, G7_)     \
            MOE_STEP(st2, st3, st1, af0, af1, NA_, NB_, BOFF_, MF_, G4_, G5_, G6_, G7_)     \
            MOE_STEP(st3, st0, st2, af1, af0, NA_, NB_, BOFF_, MF_, G4_, G5_, G6_, G7_)     \
        }                                                                                   \
    }

    int kt = kt0;
    if (kt0 < kt1) {
        // Only the 16-row fragments that hold some of the tile's rows are
        // multiplied (the rest stay zero and are never stored): a tail tile
        // (the expert's last 1..128 rows, the same rows in every wave) takes
        // 2, 4, 6 or 8 of them, a full tile with at most 192 rows 6 per wave.
        // MOE_K_LOOP(A loads and B loads per lane and step, B's offset in a
        // stage, fragments per wave, bytes between a wave's fragments in a
        // stage, DMA loads placed among MFMA groups 4..7).
        const int tile_rows = min(row_end - row0, 256);
        if (!is_tail) {
            if (tile_rows <= 192) MOE_K_LOOP(4, 4, kBOffFull, 6, 32 * 64, 2, 2, 2, 2)
            else MOE_K_LOOP(4, 4, kBOffFull, 8, 32 * 64, 2, 2, 2, 2)
        } else {
            if (tile_rows <= 32) MOE_K_LOOP(2, 8, kBOffTail, 2, 16 * 64, 0, 0, 0, 0)
            else if (tile_rows <= 64) MOE_K_LOOP(2, 8, kBOffTail, 4, 16 * 64, 0, 0, 0, 0)
            else if (tile_rows <= 96) MOE_K_LOOP(2, 8, kBOffTail, 6, 16 * 64, 3, 3, 2, 2)
            else MOE_K_LOOP(2, 8, kBOffTail, 8, 16 * 64, 3, 3, 2, 2)
        }
    }
#undef MOE_K_LOOP
#undef MOE_SCHED_GROUP
#undef MOE_SCHED_GROUP6
#undef MOE_MFMAS
#undef MOE_READ_B
#undef MOE_READ_A
#undef MOE_STEP
#undef MOE_ISSUE_STAGE
    // No load may still be writing LDS when the stages are reused below.
    MOE_WAIT_VM(0);

    if (DUAL) {
        tile_epilogue<DUAL>(acc, geo, C, R, N, kb, st0, st1);
        return;
    }
    // GEMM 2: one store loop for both cases, so the accumulators go out
    // in one pass with no branch between two store paths.  A whole tile
    // writes fp32 y; a K piece writes its fp32 partial sums to its slot,
    // laid out as the tile itself, row-major: 256 rows x 256 columns, or
    // 128 rows x 512 columns (both column tiles) for a tail tile.
    float* dst;
    int stride, rlim, clim;
    if (piece < 0) {
        dst = reinterpret_cast<float*>(C) + (size_t)row0 * N + col0;
        stride = N;
        rlim = row_end - row0;
        clim = N - col0;
    } else {
        const int first_slot = piece_bases.slot + rt * sc.p;
        if (piece == 0 && threadIdx.x == 0) {
            int* desc = reinterpret_cast<int*>(partials) + 64 + 8 * (piece_bases.cut + rt);
            desc[0] = row0;
            desc[1] = row_end;
            desc[2] = col0;
            desc[3] = is_tail ? 1 : 0;
            desc[4] = first_slot;
            desc[5] = sc.p;
        }
        dst = partials + kHeaderFloats + (size_t)(first_slot + piece) * kSlotFloats;
        stride = is_tail ? 512 : 256;
        rlim = 1 << 30;
        clim = 1 << 30;
    }
    // The lane terms are formed afresh here (wave index as a scalar, lane
    // from mbcnt) rather than reused from before the K loop, where keeping
    // them would cost registers across it.
    const int ewave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int elane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int rbase = (is_tail ? 0 : (ewave >> 1) * 16) + 4 * (elane >> 4);
    const int mstride = is_tail ? 16 : 32;  // tile rows from one fragment to the next
    const int cbase = (is_tail ? (ewave >> 1) * BN : 0) + (ewave & 1) * 128 + (elane & 15);
#pragma unroll
    for (int m = 0; m < 8; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = rbase + mstride * m + r;
            if (row >= rlim) continue;
#pragma unroll
            for (int n = 0; n < 8; ++n) {
                const int col = cbase + 16 * n;
                if (col < clim) dst[(size_t)row * stride + col] = acc[m][n][r];
            }
        }
}

// GEMM 2's tiles cut into K pieces: sum the pieces' partial sums in piece
// order and store y.  Elementwise over the cut tiles (their descriptors come
// from the header): work unit = (cut tile, 256 float4 of its row-major sums),
// so loads and y stores are 16-byte, row-contiguous and coalesced, and the
// loads of every piece are in flight together.
__global__ __launch_bounds__(kThreads) void tile_fixup_kernel(const float* __restrict__ partials,
                                                              float* __restrict__ y, int N) {
    constexpr int UNITS = kSlotFloats / 4 / kThreads;  // 64 work units per cut tile
    const int* hdr = reinterpret_cast<const int*>(partials);
    int n_cut = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) n_cut += hdr[8 * x];
    for (int w = blockIdx.x; w < n_cut * UNITS; w += gridDim.x) {
        const int g = w / UNITS;  // cut tile
        const int c = w - g * UNITS;
        const int* desc = hdr + 64 + 8 * g;
        const int row0 = desc[0], row_end = desc[1], col0 = desc[2], is_tail = desc[3];
        const int first_slot = desc[4], p = desc[5];
        const float4* src = reinterpret_cast<const float4*>(partials + kHeaderFloats) +
                            (size_t)first_slot * (kSlotFloats / 4);
        const int i = c * kThreads + threadIdx.x;  // float4 of the tile
        float4 a = src[i];
        for (int j = 1; j < p; ++j) {
            const float4 v = src[(size_t)j * (kSlotFloats / 4) + i];
            a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
        }
        const int width4 = is_tail ? 128 : 64;  // float4 per tile row
        const int grow = row0 + i / width4;
        const int gc = col0 + 4 * (i % width4);
        if (grow < row_end && gc < N) *reinterpret_cast<float4*>(y + (size_t)grow * N + gc) = a;
    }
}

// Workgroups of a persistent launch: the current device's CU count, rounded
// down to a multiple of 8 (queried once per device).
int cus_per_xcd() {
    static std::atomic<int> cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return kMaxCpx;
    int c = cached[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 8 * kMaxCpx;
        c = n / 8;
        if (c < 1) c = 1;
        if (c > kMaxCpx) c = kMaxCpx;
        cached[dev].store(c, std::memory_order_relaxed);
    }
    return c;
}

template <bool DUAL, bool NT_B>
hipError_t launch_tile(const void* A, const void* B0, const void* B1, void* C, float* partials,
                       const int32_t* offsets, int R, int E, int K, int N, int kb,
                       hipStream_t stream) {
    const long long BN = DUAL ? 128 : 256;
    const long long NT = (N + BN - 1) / BN;
    // bound on the tile count: per expert at most ceil(n_e / 256) row tiles
    // per column tile (a tail tile covers two column tiles)
    const long long mtiles = (R + kBM - 1) / kBM + E;
    const long long n_max = mtiles * NT;
    const int cpx = cus_per_xcd();
    // GEMM 1 tiles are never cut: the SwiGLU fixup of cut tiles cost more than
    // the rounds it saved (measured at T = 1024 .. 4096).
    const int max_pieces = DUAL ? 1 : kMaxPieces;
    // per XCD: its eighth of the tiles, plus at most 2 cpx extra pieces when
    // tiles may be cut (a workgroup past the XCD's items exits at once, but
    // still waits for a free CU: its LDS is a whole CU's)
    const long long grid = 8 * ((n_max + 7) / 8 + (max_pieces > 1 ? 2 * cpx : 0));
    hipLaunchKernelGGL((tile_gemm_kernel<DUAL, NT_B>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                       reinterpret_cast<const bf16*>(A), reinterpret_cast<const bf16*>(B0),
                       reinterpret_cast<const bf16*>(B1), C, partials, offsets, R, E, K, N, cpx, max_pieces, kb);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || DUAL) return err;
    // GEMM 2's cut tiles: at most 8 (cpx - 1) of 64 units each, one
    // workgroup per unit (the ones past the cut tiles exit at once)
    const unsigned fix_grid = (unsigned)(8 * cpx * (kSlotFloats / 4 / kThreads));
    hipLaunchKernelGGL(tile_fixup_kernel, dim3(fix_grid), dim3(kThreads), 0, stream, partials,
                       reinterpret_cast<float*>(C), N);
    return hipGetLastError();
}

}  // namespace

// GEMM 1 with its weight DMA marked nontemporal (gemm_tile_nt.hip).
hipError_t launch_gemm1_swiglu_tile_nt(const void* x_perm, const void* w1, const void* w3,
                                       const int32_t* offsets, int R, int E, int d, int f, int kb,
                                       float* partials, void* h, hipStream_t stream);

}  // namespace moe
