// tile_order.h -- the numbering of the 256-row macro tiles of the tile GEMMs
// (gemm_tile.hip): which expert, rows and column tile tile number t covers,
// from the per-expert row offsets alone.
//
// Tiles are numbered by expert, then groups of kGroupPairs pairs of column
// tiles; within a group, the full-row tiles in blocks of kRowBlock row tiles
// (rows fastest, then the group's columns), then the group's tail tiles, one
// per pair.  An XCD's round of 32 tiles on an expert with many rows is then 8
// row tiles x 4 column tiles, which read 8 A slabs and 4 weight slabs per K
// step from its L2 (32 row tiles of one column tile would read 33).
//
// Plain functions of their arguments: the kernels call them on the device,
// and the CPU tests compile this header with a host compiler to check that
// the numbering covers every tile exactly once.
#pragma once

#include <cstdint>

#if defined(__HIP__)
#define MOE_TILE_FN __host__ __device__ __attribute__((always_inline)) inline
#else
#define MOE_TILE_FN inline
#endif

namespace moe {

constexpr int kBM = 256;        // rows of a full tile
constexpr int kGroupPairs = 2;  // pairs of column tiles per group
constexpr int kRowBlock = 8;    // row tiles per block within a group

MOE_TILE_FN int tile_min(int a, int b) { return a < b ? a : b; }

// Geometry of tile t, in the order above.  Per expert with n_e rows: mt_n
// row tiles of 256 (the last one partial when more than 128 rows remain) per
// column tile, plus one tail tile per pair of column tiles when 1..128 rows
// remain.
struct TileGeo {
    int e, row0, row_end, col0;
    bool is_tail;
};

MOE_TILE_FN int count_tiles(const int32_t* offsets, int E, int NT, int NTP) {
    int n = 0;
    for (int e = 0; e < E; ++e) {
        const int n_e = offsets[e + 1] - offsets[e];
        const int rem = n_e & (kBM - 1);
        const int mt_n = (n_e >> 8) + (rem > 128 ? 1 : 0);
        const int tail = (rem > 0 && rem <= 128) ? 1 : 0;
        n += mt_n * NT + tail * NTP;
    }
    return n;
}

MOE_TILE_FN TileGeo tile_geometry(int t, const int32_t* offsets, int E, int NT, int NTP,
                                  int BN) {
    TileGeo g{0, 0, 0, 0, false};
    int L = t;
    for (int e = 0; e < E; ++e) {
        const int o0 = offsets[e];
        const int n_e = offsets[e + 1] - o0;
        const int rem = n_e & (kBM - 1);
        const int mt_n = (n_e >> 8) + (rem > 128 ? 1 : 0);
        const int tail = (rem > 0 && rem <= 128) ? 1 : 0;
        const int per_e = mt_n * NT + tail * NTP;
        if (L < per_e) {
            // group q of up to kGroupPairs pairs of column tiles (the last
            // group may hold fewer, and its last pair one column tile when NT
            // is odd): its full-row tiles in blocks of kRowBlock row tiles,
            // rows fastest, then the group's tail tiles, one per pair
            const int full_group = mt_n * 2 * kGroupPairs + tail * kGroupPairs;
            const int q = tile_min(L / full_group, (NTP - 1) / kGroupPairs);
            const int r = L - q * full_group;
            const int c_first = 2 * kGroupPairs * q;                     // first column tile
            const int n_cols = tile_min(2 * kGroupPairs, NT - c_first);  // column tiles in the group
            g.e = e;
            if (r < mt_n * n_cols) {
                const int b = r / (n_cols * kRowBlock);
                const int w = r - b * n_cols * kRowBlock;
                const int nb = tile_min(kRowBlock, mt_n - b * kRowBlock);  // row tiles in the block
                g.col0 = (c_first + w / nb) * BN;
                g.row0 = o0 + (b * kRowBlock + w % nb) * kBM;
            } else {
                g.is_tail = true;
                g.col0 = (c_first + 2 * (r - mt_n * n_cols)) * BN;
                g.row0 = o0 + (n_e >> 8) * kBM;
            }
            g.row_end = o0 + n_e;
            return g;
        }
        L -= per_e;
    }
    return g;
}

}  // namespace moe
