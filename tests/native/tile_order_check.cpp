// tile_order_check.cpp -- the tile GEMMs' tile numbering (tile_order.h),
// compiled for the host and checked on random expert row counts: every tile
// number maps to a valid tile, no two numbers to the same tile, and every
// tile an expert needs (its full-row tiles in every column tile, and one tail
// tile per pair of column tiles when 1..128 rows remain past its last
// multiple of 256) is covered.  Also checks the round shape the order is
// for: on an expert of 20 row tiles and 12 column tiles, each run of 32
// tiles of its first band that starts at a column boundary is 8 row tiles x
// 4 column tiles, the same 8 row tiles in every run, and any other run of
// 32 in the band spans those 8 row tiles and 5 column tiles.  Prints "ok" and exits 0 on success.
#include <cstdio>
#include <random>
#include <set>
#include <tuple>

#include "tile_order.h"

using moe::TileGeo;

static int check_one(const int32_t* off, int E, int NT, int BN, long* checked) {
    const int NTP = (NT + 1) / 2;
    const int n = moe::count_tiles(off, E, NT, NTP);
    std::set<std::tuple<int, int, int, int>> seen;
    for (int t = 0; t < n; ++t) {
        const TileGeo g = moe::tile_geometry(t, off, E, NT, NTP, BN);
        const int n_e = off[g.e + 1] - off[g.e];
        if (g.e < 0 || g.e >= E || g.row_end != off[g.e + 1] || g.row0 < off[g.e] ||
            g.row0 >= g.row_end || (g.row0 - off[g.e]) % moe::kBM != 0 || g.col0 % BN != 0 ||
            g.col0 / BN >= NT) {
            std::printf("tile %d: bad geometry\n", t);
            return 1;
        }
        const int rem = n_e % moe::kBM;
        if (g.is_tail && (!(rem > 0 && rem <= 128) || g.row0 != off[g.e] + (n_e / moe::kBM) * moe::kBM ||
                          (g.col0 / BN) % 2 != 0)) {
            std::printf("tile %d: bad tail tile\n", t);
            return 1;
        }
        if (!seen.insert(std::make_tuple(g.e, g.row0, g.col0, (int)g.is_tail)).second) {
            std::printf("tile %d: numbered twice\n", t);
            return 1;
        }
    }
    long want = 0;
    for (int e = 0; e < E; ++e) {
        const int n_e = off[e + 1] - off[e], rem = n_e % moe::kBM;
        const int mt = n_e / moe::kBM + (rem > 128 ? 1 : 0);
        const bool tail = rem > 0 && rem <= 128;
        want += (long)mt * NT + (tail ? NTP : 0);
        for (int m = 0; m < mt; ++m)
            for (int c = 0; c < NT; ++c)
                if (!seen.count(std::make_tuple(e, off[e] + m * moe::kBM, c * BN, 0))) {
                    std::printf("expert %d: row tile %d, column tile %d missing\n", e, m, c);
                    return 1;
                }
        if (tail)
            for (int p = 0; p < NTP; ++p)
                if (!seen.count(std::make_tuple(e, off[e] + (n_e / moe::kBM) * moe::kBM, 2 * p * BN, 1))) {
                    std::printf("expert %d: tail tile of pair %d missing\n", e, p);
                    return 1;
                }
    }
    if (want != n || (long)seen.size() != n) {
        std::printf("tile count %d, expected %ld\n", n, want);
        return 1;
    }
    *checked += n;
    return 0;
}

int main() {
    std::mt19937 rng(12345);
    long checked = 0;
    for (int trial = 0; trial < 3000; ++trial) {
        const int E = 1 + (int)(rng() % 9);
        const int NT = 1 + (int)(rng() % 120);
        int32_t off[10];
        off[0] = 0;
        for (int e = 0; e < E; ++e) {
            const int mode = (int)(rng() % 4);
            const int n = mode == 0   ? (int)(rng() % 300)
                          : mode == 1 ? (int)(rng() % 3000)
                          : mode == 2 ? (int)(rng() % 60) * 256 + (int)(rng() % 3) * 64
                                      : (int)(rng() % 20000);
            off[e + 1] = off[e] + n;
        }
        if (check_one(off, E, NT, trial % 2 ? 128 : 256, &checked)) return 1;
    }
    // round shape: an expert of 20 row tiles, 12 column tiles (first band:
    // tiles 0..95, rows 0..7)
    const int32_t off[2] = {0, 20 * 256};
    for (int start : {0, 32, 64, 16, 4, 20, 44}) {
        std::set<int> rows, cols;
        for (int t = start; t < start + 32; ++t) {
            const TileGeo g = moe::tile_geometry(t, off, 1, 12, 6, 128);
            rows.insert(g.row0 / 256);
            cols.insert(g.col0 / 128);
        }
        // (a run that starts part way through a column ends part way
        // through its fifth)
        const size_t want_cols = start % 8 ? 5 : 4;
        if (rows.size() != 8 || *rows.begin() != 0 || *rows.rbegin() != 7 ||
            cols.size() != want_cols) {
            std::printf("tiles %d..%d span %zu row tiles x %zu column tiles, expected rows 0..7 x %zu\n",
                        start, start + 31, rows.size(), cols.size(), want_cols);
            return 1;
        }
    }
    std::printf("ok: %ld tiles checked\n", checked);
    return 0;
}
