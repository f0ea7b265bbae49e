// schedule_dump.cpp -- prints csrc/tile_order.h's XCD schedule, compiled for
// the host, for the inputs read from stdin ("n_tiles cpx KT max_pieces" per
// line): per XCD "start full r p slot cut".  tests/test_tile_order.py
// compares it with the tests' own statement of the schedule.
#include <cstdio>

#include "tile_order.h"

int main() {
    int n, cpx, kt, mp;
    while (std::scanf("%d %d %d %d", &n, &cpx, &kt, &mp) == 4) {
        for (int x = 0; x < 8; ++x) {
            const moe::XcdSched s = moe::xcd_schedule(n, x, cpx, kt, mp);
            const moe::XcdBases b = moe::xcd_bases(n, x, cpx, kt, mp);
            std::printf("%d %d %d %d %d %d\n", s.start, s.full, s.r, s.p, b.slot, b.cut);
        }
    }
    return 0;
}
