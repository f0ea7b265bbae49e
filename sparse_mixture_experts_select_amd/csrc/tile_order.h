// tile_order.h -- the numbering of the 256-row macro tiles of the tile GEMMs
// (tile_gemm.h): which expert, rows and column tile tile number t covers,
// from the per-expert row offsets alone.
//
// Tiles are numbered by expert, then bands of kRowBlock full row tiles (the
// last band of an expert takes its remaining full rows and its tail row);
// within a band, pairs of column tiles in order, and within a pair the
// band's full-row tiles, rows fastest, column by column, then the pair's
// tail tile.  An XCD's round of 32 tiles on an expert with many rows is then
// 8 row tiles x 4 column tiles, and a round that straddles two groups of
// columns still reads the same 8 A slabs (8 slabs + 5 weight panels per K
// step from its L2; an order in blocks of 8 rows x 4 columns, rows first,
// makes straddling rounds read 16 slabs + 4 panels).
//
// Also the schedule of a launch's tiles over the 8 XCDs (xcd_schedule): each
// XCD's run of tile numbers, and how GEMM 2 cuts the tiles of an XCD's last,
// partial round into K pieces.
//
// Plain functions of their arguments: the kernels call them on the device,
// and the CPU tests compile this header with a host compiler to check that
// the numbering covers every tile exactly once and to compare the schedule
// with the tests' own statement of it.
#pragma once

#include <cstdint>

#if defined(__HIP__)
#define MOE_TILE_FN __host__ __device__ __attribute__((always_inline)) inline
#else
#define MOE_TILE_FN inline
#endif

namespace moe {

constexpr int kBM = 256;      // rows of a full tile
constexpr int kRowBlock = 8;  // full row tiles per band

constexpr int kMaxCpx = 32;         // CUs per XCD the schedule plans for (MI355X: 32)
constexpr int kMaxPieces = 8;       // K pieces per cut tile (GEMM 2)
constexpr int kPieceOverhead = 16;  // per-item cost in K steps: pipeline fill, epilogue
constexpr int kPieceTraffic = 1;    // per-piece cost in K steps: its 256 KiB partial sum
                                    // written and read back by the fixup (measured)

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
            // n_band bands of kRowBlock rows, then the last band: the
            // remaining full rows (a whole kRowBlock when they divide evenly
            // and there is no tail) and the tail row
            int n_band = mt_n / kRowBlock;
            int last_rows = mt_n - n_band * kRowBlock;
            if (last_rows == 0 && !tail) {
                n_band -= 1;
                last_rows = kRowBlock;
            }
            int b, lb, nr, th;
            if (L < n_band * kRowBlock * NT) {
                b = L / (kRowBlock * NT);
                lb = L - b * kRowBlock * NT;
                nr = kRowBlock;
                th = 0;
            } else {
                b = n_band;
                lb = L - n_band * kRowBlock * NT;
                nr = last_rows;
                th = tail;
            }
            // pair p of the band: its nr x (1 or 2) full-row tiles, rows
            // fastest, then its tail tile (the last pair holds one column
            // tile when NT is odd)
            const int per_pair = 2 * nr + th;
            const int p = tile_min(lb / per_pair, NTP - 1);
            const int r = lb - p * per_pair;
            const int n_cols = tile_min(2, NT - 2 * p);
            g.e = e;
            if (r < nr * n_cols) {
                g.col0 = (2 * p + r / nr) * BN;
                g.row0 = o0 + (b * kRowBlock + r % nr) * kBM;
            } else {
                g.is_tail = true;
                g.col0 = 2 * p * BN;
                g.row0 = o0 + (n_e >> 8) * kBM;
            }
            g.row_end = o0 + n_e;
            return g;
        }
        L -= per_e;
    }
    return g;
}

// Work of XCD x.  Workgroup IDs are dealt to the 8 XCDs round-robin, so XCD
// x runs the workgroups with blockIdx % 8 == x; it gets the x-th run of
// ceil(n/8) tile numbers (tiles sharing a weight panel then share one L2).  Its
// first `full` tiles, whole rounds of its cpx CUs, run whole; the r left over
// (fewer than cpx) are each cut into p equal K ranges when that finishes the
// XCD's work sooner (fewer idle CUs in its last round), the pieces of one K
// range of all r tiles running together.  KT: K steps of a tile.
struct XcdSched {
    int start, full, r, p;
};

MOE_TILE_FN XcdSched xcd_schedule(int n_tiles, int x, int cpx, int KT, int max_pieces) {
    XcdSched s;
    const int per_xcd = (n_tiles + 7) / 8;
    s.start = tile_min(x * per_xcd, n_tiles);
    const int n_x = tile_min(s.start + per_xcd, n_tiles) - s.start;
    s.full = (n_x / cpx) * cpx;
    s.r = n_x - s.full;
    s.p = 1;
    if (s.r > 0) {
        int best = (KT + kPieceOverhead);  // one round of whole tiles
        for (int p = 2; p <= max_pieces; ++p) {
            if (s.r * p > 2 * cpx || KT / p < 8) break;
            const int cost = ((s.r * p + cpx - 1) / cpx) * ((KT + p - 1) / p + kPieceOverhead) +
                             s.r * p * kPieceTraffic;
            if (cost < best) {
                best = cost;
                s.p = p;
            }
        }
    }
    return s;
}

// First partial-sum slot and first cut-tile number of XCD x (the XCDs'
// pieces and cut tiles are packed in XCD order).
struct XcdBases {
    int slot, cut;
};

MOE_TILE_FN XcdBases xcd_bases(int n_tiles, int x, int cpx, int KT, int max_pieces) {
    XcdBases b{0, 0};
    for (int x2 = 0; x2 < x; ++x2) {
        const XcdSched s = xcd_schedule(n_tiles, x2, cpx, KT, max_pieces);
        if (s.p > 1) {
            b.slot += s.r * s.p;
            b.cut += s.r;
        }
    }
    return b;
}

}  // namespace moe
