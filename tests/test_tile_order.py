"""The tile GEMMs' tile numbering (csrc/tile_order.h), built for the host and
checked on the CPU: every tile covered exactly once, and rounds of 8 row tiles
x 4 column tiles on experts with many rows."""
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
