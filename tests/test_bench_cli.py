"""bench.py's command-line contract that needs no GPU: a run on more than
one GPU is refused with a message, and the per-stage roofline figures are
computed from the stages' algorithmic work."""
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode != 0
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""


def test_stage_rooflines_use_algorithmic_work():
    sys.path.insert(0, ROOT)
    import bench
    from sparse_mixture_experts_select_amd import inputs
    wl = inputs.WORKLOADS["prefill"]
    counts = np.full(wl.E, wl.T * wl.k // wl.E)
    st = bench.stage_rooflines(wl, counts, {"gather_rows": 0.02, "gemm1_swiglu": 2.0,
                                            "route_scan": 0.01}, decode=False)
    R = wl.T * wl.k
    # gather: every grouped row read and written once, in bf16
    assert st["gather_rows"]["bound"] == "hbm"
    assert abs(st["gather_rows"]["achieved"] - 2 * R * wl.d * 2 / 0.02e-3 / 1e9) < 1.0
    # GEMM 1: 4 R d f flops
    assert st["gemm1_swiglu"]["bound"] == "mfma"
    assert abs(st["gemm1_swiglu"]["achieved"] - 4.0 * R * wl.d * wl.f / 2e-3 / 1e12) < 0.1
    assert st["route_scan"] == {"bound": "latency", "ms": 0.01}


def test_design_traffic_counts_intermediates():
    sys.path.insert(0, ROOT)
    import bench
    from sparse_mixture_experts_select_amd import inputs
    wl = inputs.WORKLOADS["prefill"]
    R = wl.T * wl.k
    # x_perm and h in bf16, y in fp32, each written once and read once
    assert bench.design_traffic(wl, True) == 4 * R * (wl.d + wl.f) + 8 * R * wl.d
    assert bench.design_traffic(wl, False) == 4 * R * wl.f + 8 * R * wl.d
