"""The tile GEMMs' tile numbering (csrc/tile_order.h), built for the host and
checked on the CPU: every tile covered exactly once, and rounds of 8 row tiles
x 4 column tiles, bands keeping their 8 row tiles, on experts with many rows."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_mixture_experts_select_amd", "csrc")


def test_tile_numbering_covers_every_tile_once(tmp_path):
    exe = tmp_path / "tile_order_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(ROOT, "tests", "native", "tile_order_check.cpp"), "-o", str(exe)],
                   check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok"), res.stdout


def test_xcd_schedule_matches_the_tests_statement(tmp_path):
    """The per-XCD schedule and the partial-sum slot bases of tile_order.h,
    compiled for the host, against tests/tile_plan.py on random launches."""
    import random

    import tile_plan
    exe = tmp_path / "schedule_dump"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(ROOT, "tests", "native", "schedule_dump.cpp"), "-o", str(exe)],
                   check=True)
    rng = random.Random(7)
    cases = [(rng.randint(1, 5000), rng.choice([1, 7, 16, 32]), rng.randint(1, 600),
              rng.choice([1, 2, 8])) for _ in range(400)]
    cases += [(8, 32, 64, 8), (8, 32, 48, 8), (8, 32, 40, 8), (264, 32, 64, 8)]
    inp = "".join("%d %d %d %d\n" % c for c in cases)
    res = subprocess.run([str(exe)], input=inp, capture_output=True, text=True, timeout=60, check=True)
    lines = res.stdout.split("\n")
    i = 0
    for n, cpx, kt, mp in cases:
        slot = cut = 0
        for x in range(8):
            start, full, r, p = tile_plan.xcd_schedule(n, x, cpx, kt, mp)
            got = list(map(int, lines[i].split()))
            assert got == [start, full, r, p, slot, cut], ((n, cpx, kt, mp, x), got)
            if p > 1:
                slot += r * p
                cut += r
            i += 1
