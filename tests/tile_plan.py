"""The tile GEMMs' plan written out independently for the tests: how many
256-row tiles a launch has and how the per-XCD schedule cuts GEMM 2's last
round into K pieces (the kernels take these from csrc/tile_order.h;
tests/test_tile_order.py checks this statement against that header compiled
for the host).  Used to choose parity cases that reach given piece counts."""
from __future__ import annotations

BM = 256
MAX_PIECES = 8
PIECE_OVERHEAD = 16
PIECE_TRAFFIC = 1


def count_tiles(counts, NT):
    """Tiles for experts with these row counts and NT column tiles: per
    expert, whole 256-row tiles (a last partial one when more than 128 rows
    remain) in every column tile, plus one tail tile per pair of column
    tiles when 1..128 rows remain."""
    NTP = (NT + 1) // 2
    n = 0
    for n_e in counts:
        rem = n_e % BM
        mt = n_e // BM + (1 if rem > 128 else 0)
        n += mt * NT + (NTP if 0 < rem <= 128 else 0)
    return n


def xcd_schedule(n_tiles, x, cpx, KT, max_pieces=MAX_PIECES):
    """(start, full, r, p) of XCD x: its run of ceil(n/8) tiles, the whole
    rounds of cpx, the r left over and the number of K pieces p each of them
    is cut into (1: not cut), the p that minimises the XCD's cost in K steps
    (rounds x (K steps per piece + overhead) + the pieces' partial sums),
    with at most 2 cpx pieces and at least 8 K steps per piece."""
    per = (n_tiles + 7) // 8
    start = min(x * per, n_tiles)
    n_x = min(start + per, n_tiles) - start
    full = (n_x // cpx) * cpx
    r = n_x - full
    p_best = 1
    if r > 0:
        best = KT + PIECE_OVERHEAD
        for p in range(2, max_pieces + 1):
            if r * p > 2 * cpx or KT // p < 8:
                break
            cost = -(-r * p // cpx) * (-(-KT // p) + PIECE_OVERHEAD) + r * p * PIECE_TRAFFIC
            if cost < best:
                best, p_best = cost, p
    return start, full, r, p_best


def gemm2_pieces(counts, d, f, cpx=32):
    """The set of piece counts GEMM 2 (K = f, 256-column tiles over d) cuts
    tiles into, for experts with these row counts."""
    n = count_tiles(counts, (d + 255) // 256)
    out = set()
    for x in range(8):
        _, _, r, p = xcd_schedule(n, x, cpx, f // 32)
        if r > 0 and p > 1:
            out.add(p)
    return out
