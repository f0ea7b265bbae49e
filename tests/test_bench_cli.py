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


def test_source_digest_ignores_comments_only(tmp_path, monkeypatch):
    """The digest that keys the committed counter figures changes with the
    kernels' code, not with an edit of their comments or layout."""
    sys.path.insert(0, ROOT)
    import bench
    names = ("tile_gemm.h", "common.h", "tile_order.h", "gemm_tile.hip")
    for n in names:
        (tmp_path / n).write_text(open(os.path.join(bench.CSRC, n)).read())
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    base = bench.source_digest("prefill")
    f = tmp_path / "tile_gemm.h"
    text = f.read_text()
    f.write_text("// a new leading comment\n" + text.replace("\n", "\n\n", 3) + "\n/* and a block */\n")
    assert bench.source_digest("prefill") == base
    f.write_text(text.replace("constexpr int kBK = 32;", "constexpr int kBK = 64;"))
    assert bench.source_digest("prefill") != base


def test_summarize_stalls_on_synthetic_counters(tmp_path, monkeypatch):
    """The wave-state summary from four counter passes: per kernel the
    counters averaged over launches and the fractions formed from them."""
    sys.path.insert(0, ROOT)
    import csv
    import bench
    g1 = "_ZN3moe12_GLOBAL__N_116tile_gemm_kernelILb1ELb0EEEvPKDF16b"
    g2 = "_ZN3moe12_GLOBAL__N_116tile_gemm_kernelILb0ELb1EEEvPKDF16b"
    values = {"SQ_WAVE_CYCLES": 1000.0, "SQ_WAIT_ANY": 150.0, "SQ_WAIT_INST_ANY": 400.0,
              "SQ_ACTIVE_INST_ANY": 450.0, "SQ_VALU_MFMA_BUSY_CYCLES": 2400.0,
              "SQ_LDS_BANK_CONFLICT": 10.0, "SQ_INSTS_LDS": 1000.0, "SQ_INSTS_MFMA": 640.0,
              "SQ_INSTS_VALU": 700.0, "SQ_INSTS_SALU": 200.0, "SQ_INSTS_VMEM": 80.0,
              "SQ_WAVES": 10.0, "GRBM_GUI_ACTIVE": 8 * 2.0e6}
    dirs = []
    passes = [p.split() for p in bench.STALL_PASSES]
    for i, counters in enumerate(passes):
        d = tmp_path / ("p%d" % i)
        d.mkdir()
        with open(d / "run_counter_collection.csv", "w", newline="") as fh:
            w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                                "Counter_Value", "Start_Timestamp", "End_Timestamp"])
            w.writeheader()
            for disp, name in ((1, g1), (2, g2), (3, g1)):
                for c in counters + ["GRBM_GUI_ACTIVE"]:
                    w.writerow({"Dispatch_Id": disp, "Kernel_Name": name, "Counter_Name": c,
                                "Counter_Value": values.get(c, 1.0), "Start_Timestamp": 0,
                                "End_Timestamp": 1000000})  # 1 ms
        dirs.append(str(d))
    (tmp_path / "profiles").mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    bench.summarize_stalls(dirs)
    text = (tmp_path / "profiles" / "tile_gemm_prefill_wave_states.txt").read_text()
    assert "[w1/w3 grouped GEMM + SwiGLU]" in text and "[w2 grouped GEMM]" in text
    assert "clock_ghz_from_grbm = 2.000" in text           # 16e6 / 8 / 1 ms
    assert "waiting_on_waitcnt_or_barrier = 0.150" in text  # 150 / 1000
    assert "ready_but_not_issued = 0.400" in text
    assert "mfma_busy_of_wave_cycles = 0.600" in text       # 2400 / (4 x 1000)
    assert "per wave: mfma 64," in text
