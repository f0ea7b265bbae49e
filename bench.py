"""Benchmark of the MoE feed-forward layer on one MI355X.

Prints ONE JSON line on stdout.  A step is one full layer call
(router + top-k/softmax, grouping, both grouped GEMMs, combine) over one batch
of synthetic inputs that are already resident in HBM.  The primary workload is
the T=32 decode batch at Mixtral shapes (d=4096, f=14336, E=8, k=2, bf16),
which is HBM-bound; the T=4096 prefill batch (MFMA-bound) is reported beside
it under "secondary", the T=16384 batch with skewed routing under "skewed"
and the 32-block stack under "stack".

Live timing: the K timed steps are bracketed by torch.cuda.synchronize();
inside them the library records HIP events on the launch stream just before
and just after the dominant kernel (the w1/w3 grouped GEMM with the SwiGLU
epilogue; moe_ffn_profile_begin/end), which gives its average duration over
the timed region for the roofline entry.  A further, untimed pass records
events at every stage boundary for the per-stage breakdown ("stages_ms";
each boundary event adds a few microseconds there), and another records HIP
events around each step for the per-step median, minimum and 90th percentile
("step_ms").

The CPU baseline times the fp64 oracle on the host on a bounded sample of the
same workload.  Beside the layer the line carries the measured ceilings of this
part (the read probe over the decode layer's own weights, the MFMA probe), the
prefill experts' GEMM products timed with torch.matmul for comparison
("vendor_gemm"; nothing in the layer calls it) and any plan overrides set in
the environment ("plan_overrides").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE FFN tokens/s at Mixtral shapes; % MFMA peak (prefill), % HBM BW (decode)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
CSRC = os.path.join(ROOT, "sparse_mixture_experts_select_amd", "csrc")
# The w1/w3 grouped GEMM that runs for each workload: the streamed-weight
# kernel at a few rows per expert, the 256x256 tile kernel (its weight DMA
# not marked nontemporal at these sizes) at hundreds of rows per expert.
# Patterns match both the demangled and the mangled kernel name.
GEMM1_KERNEL = {
    "decode": ("gemm_stream.hip", r"stream_gemm_kernel(<true, 1>|ILb1ELi1E)"),
    "prefill": ("tile_gemm.h", r"tile_gemm_kernel(<true, false>|ILb1ELb0E)"),
    "skewed": ("tile_gemm.h", r"tile_gemm_kernel(<true, false>|ILb1ELb0E)"),
    "stack": ("tile_gemm.h", r"tile_gemm_kernel(<true, false>|ILb1ELb0E)"),
}
CALIBRATION_BYTES = 1 << 30
# Profiling commands behind the committed summaries; {out} is the rocprofv3
# output directory that the summarizer is then pointed at.
PMC_COMMAND = ("timeout -s KILL 150 rocprofv3 --pmc {counter} --output-format csv -d {out} -o run -- "
               "python3 bench.py --steps 3 --warmup 1 --stack off --skewed off --sweep off "
               "--no-cpu-baseline --calibrate-copy")
# The skewed workload runs the same w1/w3 kernel as prefill, so its counters
# come from a run of their own.
SKEWED_PMC_COMMAND = ("timeout -s KILL 150 rocprofv3 --pmc {counter} --output-format csv -d {out} "
                      "-o run -- python3 bench.py --workload skewed --secondary none --steps 3 "
                      "--warmup 1 --stack off --sweep off --no-cpu-baseline --calibrate-copy")
# The 32-block stack (T = 2048) runs the same w1/w3 kernel as prefill; in a
# run of the stack beside the decode workload (whose w1/w3 kernel is the
# streamed one) every dispatch of the tile kernel is a stack layer.
STACK_PMC_COMMAND = ("timeout -s KILL 300 rocprofv3 --pmc {counter} --output-format csv -d {out} "
                     "-o run -- python3 bench.py --secondary none --skewed off --sweep off "
                     "--steps 3 --warmup 1 --stack on --no-cpu-baseline --calibrate-copy")
MFMA_COUNTERS = "SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU_MFMA_MOPS_BF16 GRBM_GUI_ACTIVE GRBM_COUNT"
MFMA_COMMAND = ("timeout -s KILL 150 rocprofv3 --pmc " + MFMA_COUNTERS + " --output-format csv "
                "-d {out} -o run -- python3 bench.py --workload prefill --secondary none "
                "--steps 3 --warmup 1 --stack off --skewed off --sweep off --no-cpu-baseline")
SIMDS = 256 * 4          # MI355X: 256 CUs x 4 SIMDs
# Four counter passes over the prefill tile GEMMs (at most 8 SQ counters a
# pass), summarized into the wave-state breakdown.
STALL_PASSES = (
    "SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_WAIT_INST_LDS "
    "SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VMEM SQ_VALU_MFMA_BUSY_CYCLES",
    "SQ_LDS_BANK_CONFLICT SQ_LDS_ADDR_CONFLICT SQ_LDS_IDX_ACTIVE SQ_LDS_DATA_FIFO_FULL "
    "SQ_LDS_CMD_FIFO_FULL SQ_INST_LEVEL_LDS SQ_INSTS_LDS SQ_LDS_UNALIGNED_STALL",
    "SQ_VMEM_TA_ADDR_FIFO_FULL SQ_VMEM_TA_CMD_FIFO_FULL SQ_INST_LEVEL_VMEM SQ_INSTS_VMEM "
    "SQ_ACTIVE_INST_ANY SQ_ACTIVE_INST_MISC SQ_ACTIVE_INST_VALU SQ_VALU_MFMA_COEXEC_CYCLES",
    "SQ_INSTS_MFMA SQ_INSTS_SALU SQ_INSTS_VALU SQ_INSTS_SMEM SQ_ACTIVE_INST_SCA "
    "SQ_INST_CYCLES_SALU SQ_WAVES SQ_CYCLES",
)
STALL_COMMAND = ("timeout -s KILL 90 rocprofv3 --pmc {counters} GRBM_GUI_ACTIVE --output-format csv "
                 "-d {out} -o run -- python3 bench.py --workload prefill --secondary none --steps 3 "
                 "--warmup 1 --stack off --skewed off --sweep off --vendor off --no-cpu-baseline")
NOMINAL_CLOCK_HZ = 2.4e9  # the clock the 2.5 PFLOP/s figure assumes
TRACE_COMMAND = ("rocprofv3 --kernel-trace --stats --output-format csv -d {out} -o run -- "
                 "python3 bench.py --steps 10 --warmup 2 --sweep off --cpu-seconds 2 --cpu-full none")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm1_algorithmic(wl, counts):
    """Bytes and flops one gemm1_swiglu launch must move / do: w1 and w3 of
    every expert that received rows, the grouped rows of x in, h out."""
    R = wl.T * wl.k
    active = int((counts > 0).sum())
    nbytes = active * 2 * wl.d * wl.f * 2 + R * wl.d * 2 + R * wl.f * 2
    flops = 4.0 * R * wl.d * wl.f
    return nbytes, flops


def layer_algorithmic(wl, counts):
    """Per step: flops on active parameters (router + k SwiGLU experts per
    token), and bytes of active expert weights + router + x in + out."""
    active = int((counts > 0).sum())
    flops = wl.T * (2.0 * wl.d * wl.E + wl.k * 6.0 * wl.d * wl.f)
    nbytes = active * 3 * wl.d * wl.f * 2 + wl.d * wl.E * 2 + 2 * wl.T * wl.d * 2
    return flops, nbytes


def design_traffic(wl, gathered):
    """HBM bytes per layer of the intermediate tensors the design adds to
    the algorithmic traffic, each written once and read once: the grouped
    rows x_perm (bf16; only where the rows are gathered, i.e. the tile
    path), h (bf16) and y (fp32).  The streamed path writes y as a few K-slice
    partials, which adds (slices - 1) * R * d * 8 bytes, under 1% of its
    weight bytes, not counted here."""
    R = wl.T * wl.k
    parts = {"x_perm": 2 * R * wl.d * 2 if gathered else 0, "h": 2 * R * wl.f * 2,
             "y": 2 * R * wl.d * 4}
    return int(sum(parts.values()))


def stage_rooflines(wl, counts, stage_ms, decode):
    """Each stage of the layer against its own roofline, from the per-stage
    times of the breakdown pass (HIP events at the stage boundaries, so a
    stage's time includes its launch gap) and the stage's algorithmic bytes
    or flops: the router reads x and W_r and writes ids and gates; the scan
    is a latency-bound pass over T*k ids; the gather reads and writes every
    grouped row once; GEMM 1 and GEMM 2 are weight-stream bound at decode and
    MFMA bound otherwise; the combine reads one fp32 expert output per row and
    writes out."""
    R = wl.T * wl.k
    active = int((counts > 0).sum())
    hbm = {
        "router_topk": wl.T * wl.d * 2 + wl.d * wl.E * 2 + R * 8,
        "gather_rows": 2 * R * wl.d * 2,
        "combine": R * wl.d * 4 + wl.T * wl.d * 2 + R * 8,
    }
    if decode:
        hbm["gemm1_swiglu"] = active * 2 * wl.d * wl.f * 2 + R * wl.d * 2 + R * wl.f * 2
        hbm["gemm2"] = active * wl.f * wl.d * 2 + R * wl.f * 2 + R * wl.d * 4
    flops = {} if decode else {"gemm1_swiglu": 4.0 * R * wl.d * wl.f, "gemm2": 2.0 * R * wl.f * wl.d}
    out = {}
    for stage, ms in stage_ms.items():
        if stage in hbm:
            a = hbm[stage] / (ms * 1e-3) / 1e9
            # bytes that 8 TB/s moves in under 2 us: launch latency bounds it
            bound = "hbm" if hbm[stage] / (HBM_PEAK_GBS * 1e9) >= 2e-6 else "latency"
            out[stage] = {"bound": bound, "ms": ms, "achieved": round(a, 1), "unit": "GB/s",
                          "frac": round(a / HBM_PEAK_GBS, 4)}
        elif stage in flops:
            a = flops[stage] / (ms * 1e-3) / 1e12
            out[stage] = {"bound": "mfma", "ms": ms, "achieved": round(a, 1), "unit": "TFLOP/s",
                          "frac": round(a / MFMA_BF16_PEAK_TFLOPS, 4)}
        else:
            out[stage] = {"bound": "latency", "ms": ms}
    return out


def source_digest(workload):
    """Digest of the source of the w1/w3 kernel the workload runs (plus the
    headers it includes from the library), to tell whether committed counter
    figures still apply.  Comments and whitespace are left out, so an edit
    of the comments alone keeps the figures."""
    import re
    h = hashlib.sha256()
    src = GEMM1_KERNEL[workload][0]
    headers = ("common.h", "tile_order.h", "gemm_tile.hip") if src == "tile_gemm.h" else ("common.h",)
    for name in (src,) + headers:
        with open(os.path.join(CSRC, name)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def committed_traffic(workload):
    """HBM bytes per gemm1 launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "gemm1_swiglu_%s_traffic.txt" % workload)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as fh:
        for line in fh:
            if "=" in line and not line.lstrip().startswith("#"):
                key, val = line.split("=", 1)
                vals[key.strip()] = val.strip()
    if vals.get("kernel_source_sha256_16") != source_digest(workload):
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def run_workload(name, steps, warmup, binding, inputs, torch):
    wl = inputs.WORKLOADS[name]
    inp = inputs.workload_inputs(name, "cuda")
    x, wr, w1, w3, w2, bias = (inp[n] for n in ("x", "w_router", "w1", "w3", "w2", "bias"))
    out = torch.empty_like(x)
    counts = torch.zeros(wl.E, dtype=torch.int32, device="cuda")
    # one call with the routing exposed, to know which experts are active
    binding.moe_ffn_forward_ex(x, wr, w1, w3, w2, wl.k, out=out, router_bias=bias,
                               expert_counts=counts)
    torch.cuda.synchronize()
    counts_h = counts.cpu().numpy()

    def step():
        if bias is None:
            binding.moe_ffn_forward(x, wr, w1, w3, w2, wl.k, out=out)
        else:
            binding.moe_ffn_forward_ex(x, wr, w1, w3, w2, wl.k, out=out, router_bias=bias)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Timed region: events only around the w1/w3 kernel (each event costs a
    # few microseconds of GPU time).
    binding.moe_ffn_profile_begin(steps, ["gemm1_swiglu"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed_ms, calls = binding.moe_ffn_profile_end()
    assert calls == steps, (calls, steps)
    ms_per_step = 1e3 * elapsed / steps
    # Untimed breakdown pass: events at every stage boundary.
    n_bd = min(steps, 10)
    binding.moe_ffn_profile_begin(n_bd)
    for _ in range(n_bd):
        step()
    torch.cuda.synchronize()
    stage_ms, calls = binding.moe_ffn_profile_end()
    stage_avg = {kk: v / calls for kk, v in stage_ms.items() if v > 0}  # skipped stages sum to 0
    # Untimed distribution pass: HIP events around each step on the launch
    # stream (the library launches on torch's current stream).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record()
        step()
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    step_dist = {"median": round(per[len(per) // 2], 5), "min": round(per[0], 5),
                 "p90": round(per[min(len(per) - 1, int(0.9 * len(per)))], 5)}

    g_bytes, g_flops = gemm1_algorithmic(wl, counts_h)
    g_ms = timed_ms["gemm1_swiglu"] / steps
    l_flops, l_bytes = layer_algorithmic(wl, counts_h)
    res = {
        "workload": name,
        "wl": wl,
        "inp": inp,
        "ms_per_step": ms_per_step,
        "tokens_per_s": wl.T / (ms_per_step * 1e-3),
        "stage_ms": {kk: round(v, 5) for kk, v in stage_avg.items()},  # breakdown pass
        "stage_roofline": stage_rooflines(wl, counts_h, {kk: round(v, 5) for kk, v in stage_avg.items()},
                                          name == "decode"),
        "step_ms": step_dist,  # distribution pass
        "counts": counts_h.tolist(),
        "gemm1_ms": g_ms,
        "gemm1_gbs": g_bytes / (g_ms * 1e-3) / 1e9,
        "gemm1_tflops": g_flops / (g_ms * 1e-3) / 1e12,
        "gemm1_bytes": g_bytes,
        "gemm1_flops": g_flops,
        "layer_tflops": l_flops / (ms_per_step * 1e-3) / 1e12,
        "layer_gbs": l_bytes / (ms_per_step * 1e-3) / 1e9,
    }
    log("[bench] %s: %.4f ms/step, %.0f tokens/s, stages(ms) %s" %
        (name, ms_per_step, res["tokens_per_s"], res["stage_ms"]))
    return res


def run_stack(steps, warmup, binding, inputs, torch):
    """The 32-block stack h <- h + MoE(RMSNorm(h)) at T=2048 with all layers'
    weights resident.  A step restores h0 (one 16 MiB copy) and runs the 32
    blocks, one library call each (the router forms RMSNorm(h), the combine
    adds the residual in place)."""
    wl = inputs.WORKLOADS["stack"]
    layers = [inputs.make_weights(wl.d, wl.f, wl.E, torch.bfloat16, "cuda", 0, "stack", layer)
              for layer in range(wl.layers)]
    h0 = inputs.make_x(wl.T, wl.d, torch.bfloat16, "cuda", wl.x_dist, 0, "stack")
    h = torch.empty_like(h0)
    counts = [torch.zeros(wl.E, dtype=torch.int32, device="cuda") for _ in layers]
    torch.cuda.synchronize()
    log("[bench] stack: %d layers resident (%.1f GB of expert weights)"
        % (len(layers), sum(w["w1"].numel() * 3 * 2 for w in layers) / 1e9))

    def step(with_counts=False):
        h.copy_(h0)
        for i, w in enumerate(layers):
            binding.moe_ffn_forward_ex(h, w["w_router"], w["w1"], w["w3"], w["w2"], wl.k, out=h,
                                       residual=h, rmsnorm_eps=wl.rms_eps,
                                       expert_counts=counts[i] if with_counts else None)

    step(with_counts=True)
    torch.cuda.synchronize()
    active = [int((c > 0).sum().item()) for c in counts]
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    binding.moe_ffn_profile_begin(steps * wl.layers, ["gemm1_swiglu"])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed_ms, calls = binding.moe_ffn_profile_end()
    assert calls == steps * wl.layers, (calls, steps)
    ms_per_step = 1e3 * elapsed / steps
    g_ms = timed_ms["gemm1_swiglu"] / calls
    R = wl.T * wl.k
    g_flops = 4.0 * R * wl.d * wl.f
    flops = wl.layers * wl.T * (2.0 * wl.d * wl.E + wl.k * 6.0 * wl.d * wl.f)
    nbytes = sum(a * 3 * wl.d * wl.f * 2 for a in active)
    res = {
        "workload": "stack (T=%d, %d layers, d=%d, f=%d, E=%d, k=%d)"
                    % (wl.T, wl.layers, wl.d, wl.f, wl.E, wl.k),
        "value": round(wl.T / (ms_per_step * 1e-3), 1), "unit": "tokens/s",
        "ms_per_step": round(ms_per_step, 4),
        "ms_per_layer": round(ms_per_step / wl.layers, 5),
        "roofline": {"kernel": "gemm1_swiglu", "bound": "mfma",
                     "achieved": round(g_flops / (g_ms * 1e-3) / 1e12, 2),
                     "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(g_flops / (g_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                     "avg_launch_ms": round(g_ms, 5), "traffic": committed_traffic("stack")},
        "layer": {"tflops_active": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
                  "mfma_frac": round(flops / (ms_per_step * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
                  "hbm_gbs": round(nbytes / (ms_per_step * 1e-3) / 1e9, 1),
                  # every block runs the tile path (T*k/E = 512 rows per expert)
                  "design_bytes_per_layer": design_traffic(wl, True)},
    }
    # The same step replayed from one HIP graph (all 32 blocks captured;
    # the layer calls use a caller workspace, as graph capture requires).
    ws = torch.empty(binding.moe_ffn_workspace_bytes(wl.T, wl.d, wl.f, wl.E, wl.k),
                     dtype=torch.uint8, device="cuda")

    def step_ws():
        h.copy_(h0)
        for w in layers:
            binding.moe_ffn_forward_ex(h, w["w_router"], w["w1"], w["w3"], w["w2"], wl.k, out=h,
                                       residual=h, rmsnorm_eps=wl.rms_eps, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step_ws()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step_ws()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    res["graph_ms_per_step"] = round(1e3 * (time.perf_counter() - t0) / steps, 4)
    del graph
    log("[bench] stack: %.3f ms/step (%.4f ms/layer), %.0f tokens/s; one HIP graph: %.3f ms/step"
        % (ms_per_step, ms_per_step / wl.layers, res["value"], res["graph_ms_per_step"]))
    del layers
    return res


SWEEP_T = (1, 2, 4, 8, 16, 32, 64, 128, 192, 256, 320, 384, 448, 512, 768, 1024, 2048, 4096, 8192,
           16384)


def run_sweep(steps, warmup, binding, inputs, torch):
    """Tokens/s and both roofline fractions of the layer at Mixtral shapes
    over batch sizes T = 1 .. 16384 (one set of prefill-distributed weights,
    unit-RMS tokens), locating the HBM-bound to MFMA-bound crossover."""
    wl = inputs.WORKLOADS["prefill"]
    w = inputs.make_weights(wl.d, wl.f, wl.E, torch.bfloat16, "cuda", 0, "prefill", 0)
    rows = []
    for T in SWEEP_T:
        x = inputs.make_x(T, wl.d, torch.bfloat16, "cuda", "rms", 0, "sweep")
        out = torch.empty_like(x)
        counts = torch.zeros(wl.E, dtype=torch.int32, device="cuda")
        binding.moe_ffn_forward_ex(x, w["w_router"], w["w1"], w["w3"], w["w2"], wl.k, out=out,
                                   expert_counts=counts)
        torch.cuda.synchronize()
        active = int((counts > 0).sum().item())
        n = max(steps, 3)
        for _ in range(warmup):
            binding.moe_ffn_forward(x, w["w_router"], w["w1"], w["w3"], w["w2"], wl.k, out=out)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            binding.moe_ffn_forward(x, w["w_router"], w["w1"], w["w3"], w["w2"], wl.k, out=out)
        torch.cuda.synchronize()
        ms = 1e3 * (time.perf_counter() - t0) / n
        # per-stage breakdown from a separate pass (events at every boundary)
        binding.moe_ffn_profile_begin(n)
        for _ in range(n):
            binding.moe_ffn_forward(x, w["w_router"], w["w1"], w["w3"], w["w2"], wl.k, out=out)
        torch.cuda.synchronize()
        st_ms, calls = binding.moe_ffn_profile_end()
        stages = {k: round(v / max(calls, 1), 5) for k, v in st_ms.items() if v > 0}
        flops = T * (2.0 * wl.d * wl.E + wl.k * 6.0 * wl.d * wl.f)
        nbytes = active * 3 * wl.d * wl.f * 2 + wl.d * wl.E * 2 + 2 * T * wl.d * 2
        row = {"T": T, "ms": round(ms, 4), "tokens_per_s": round(T / (ms * 1e-3), 1),
               "active_experts": active,
               "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
               "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
               "hbm_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "stages_ms": stages}
        rows.append(row)
        log("[sweep] T=%5d  %8.4f ms  %11.1f tokens/s  %7.1f TFLOP/s (%.3f)  %7.1f GB/s (%.3f)"
            % (T, ms, row["tokens_per_s"], row["tflops"], row["mfma_frac"], row["hbm_gbs"],
               row["hbm_frac"]))
        log("[sweep]        stages(ms) %s" % stages)
        del x, out
    return rows


def roofline(res, bound):
    if bound == "hbm":
        achieved = res["gemm1_gbs"]
        peak, unit = HBM_PEAK_GBS, "GB/s"
    else:
        achieved = res["gemm1_tflops"]
        peak, unit = MFMA_BF16_PEAK_TFLOPS, "TFLOP/s"
    return {"kernel": "gemm1_swiglu", "bound": bound, "achieved": round(achieved, 2), "peak": peak,
            "unit": unit, "frac": round(achieved / peak, 4),
            "avg_launch_ms": round(res["gemm1_ms"], 5),
            "traffic": committed_traffic(res["workload"])}


def _host_facts():
    cpu_model, ram_gb = "unknown", None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as fh:
            for line in fh:
                if line.startswith("MemTotal"):
                    ram_gb = round(int(line.split()[1]) / 1024 ** 2, 1)
                    break
    except OSError:
        pass
    return cpu_model, ram_gb


def _oracle_full_pass(name, inputs, torch):
    """One timed pass of the oracle over every token of a workload (the
    whole layer per token, fp64, OpenMP over tokens); inputs are drawn on
    the GPU exactly as the GPU runs see them, then copied to the host."""
    import oracle
    inp = inputs.workload_inputs(name, "cuda")
    host = {n: inputs.host_array(inp[n]) for n in ("x", "w_router", "w1", "w3", "w2")}
    bias = None if inp["bias"] is None else inputs.host_array(inp["bias"])
    wl = inputs.WORKLOADS[name]
    del inp
    torch.cuda.empty_cache()
    t0 = time.perf_counter()
    oracle.moe_tokens(host["x"], host["w_router"], host["w1"], host["w3"], host["w2"], wl.k,
                      bias=bias)
    el = time.perf_counter() - t0
    log("[bench] oracle, full %s workload (%d tokens): %.2f s" % (name, wl.T, el))
    return {"tokens": wl.T, "seconds": round(el, 6), "tokens_per_s": round(wl.T / el, 3)}


def cpu_baseline(res, seconds, inputs, torch, full=("tiny", "prefill")):
    """The fp64 oracle on the host cores: the primary workload's tokens
    repeated for about `seconds` (its figure is `value`), then one pass over
    every token of each workload in `full`, each timed in full.  The skewed
    and stack workloads would take minutes (about 150 s and 600 s on 16
    cores); their times are extrapolated from the per-token cost, which is
    the same in every workload at these shapes (each token runs k experts of
    one shape)."""
    import numpy as np

    import oracle
    wl = res["wl"]
    inp = res["inp"]
    host = {n: inputs.host_array(inp[n]) for n in ("x", "w_router", "w1", "w3", "w2")}
    bias = None if inp["bias"] is None else inputs.host_array(inp["bias"])
    n_tok = min(wl.T, 32)
    tokens = np.arange(n_tok, dtype=np.int64)
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_tokens(host["x"], host["w_router"], host["w1"], host["w3"], host["w2"], wl.k,
                          tokens=tokens, bias=bias)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    del host
    tok_s = reps * n_tok / el
    cpu_model, ram_gb = _host_facts()
    per_tok = el / (reps * n_tok)
    timed = {name: _oracle_full_pass(name, inputs, torch) for name in full}
    extrap = {}
    for name in ("skewed", "stack"):
        w = inputs.WORKLOADS[name]
        extrap[name] = round(per_tok * w.T * getattr(w, "layers", 1), 1)
    return {"value": round(tok_s, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu_model": cpu_model, "ram_gb": ram_gb, "nproc": os.cpu_count(),
            "sample": "%s workload, tokens 0..%d (the whole workload; full layer per token in "
                      "fp64), %d passes, %.1f s" % (wl.name, n_tok - 1, reps, el),
            "seconds_per_token_layer": round(per_tok, 5),
            "timed_full_workloads": timed,
            "extrapolated_full_workload_seconds": extrap}


def device_facts(torch):
    """What the runtime reports for GPU 0 (compute units, ISA, memory), beside
    the 256-CU / 2.4 GHz figures the peaks assume; the clock actually held
    under load is measured separately (MFMA counter summary)."""
    p = torch.cuda.get_device_properties(0)
    return {"name": p.name, "arch": getattr(p, "gcnArchName", ""),
            "compute_units": p.multi_processor_count,
            "memory_gb": round(p.total_memory / 1e9, 1),
            "l2_bytes": getattr(p, "L2_cache_size", None)}


def read_probe(torch, binding, bufs, reps=10):
    """Measured streaming-read rate of this GPU over the very buffers the
    decode layer streams (its w1, w3 and w2, 0.94 GB each, far larger than
    the 256 MiB MALL): the library's read probe (nontemporal 16-byte loads,
    eight in flight, in a grid-stride loop), best over a few grid sizes and
    `reps` timed passes per buffer; the rate is their total bytes over the
    sum of the best times.  Reading the layer's own buffers keeps the
    comparison with GEMM 1 fair: a fresh 4 GiB buffer read at 6.8-7.2 TB/s
    from one allocation to the next."""
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    total_b, total_ms, grids = 0, 0.0, []
    for buf in bufs:
        best = None
        for blocks in (256, 384, 512, 1024):
            binding.moe_hbm_read_probe(buf, blocks, sink)
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record()
                binding.moe_hbm_read_probe(buf, blocks, sink)
                b.record()
                torch.cuda.synchronize()
                ms = a.elapsed_time(b)
                if best is None or ms < best[0]:
                    best = (ms, blocks)
        total_b += buf.numel() * buf.element_size()
        total_ms += best[0]
        grids.append(best[1])
    gbs = total_b / (total_ms * 1e-3) / 1e9
    log("[bench] read probe: %.1f GB/s (%d bytes in %d buffers, workgroups %s)"
        % (gbs, total_b, len(bufs), grids))
    return gbs, total_b, grids


def mfma_probe(torch, binding, ms_target=150.0):
    """Measured bf16 matrix-core rate of this GPU under a dense MFMA stream
    on random operands (the library's MFMA probe: the tile GEMMs' per-wave
    8 x 8 fragment shape, one workgroup of 4 waves per CU, no memory
    traffic), beside the 2.5 PFLOP/s datasheet figure, which assumes 2.4 GHz.
    Run for about ms_target milliseconds, long enough for the clock to
    settle at what the power limit allows; best of two runs, with the clock
    the probe recorded (shader cycles over 100 MHz real-time ticks)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ops = torch.randn(4 << 20, dtype=torch.float32, device="cuda").to(torch.bfloat16)  # 8 MiB
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2 * cus, dtype=torch.int64, device="cuda")

    def timed(iters):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        binding.moe_mfma_probe(ops, iters, cus, sink, clocks)
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    short = 2000
    per_iter = timed(short) / short
    iters = int(min(max(ms_target / per_iter, short), 1 << 24))
    best = None
    for _ in range(2):
        ms = timed(iters)
        ck = clocks.cpu().numpy().reshape(cus, 2).astype(float)
        ghz = ck[:, 0].sum() / ck[:, 1].sum() * 0.1
        if best is None or ms < best[0]:
            best = (ms, ghz)
    flops = cus * 4.0 * iters * 128 * 16384
    tflops = flops / (best[0] * 1e-3) / 1e12
    log("[bench] MFMA probe: %.1f TFLOP/s (%.3f of %.0f), clock %.3f GHz, %d x %d iterations"
        % (tflops, tflops / MFMA_BF16_PEAK_TFLOPS, MFMA_BF16_PEAK_TFLOPS, best[1], cus, iters))
    del ops
    torch.cuda.empty_cache()
    return {"what": "v_mfma_f32_16x16x32_bf16 on random bf16 operands, no memory traffic, one "
                    "workgroup of 4 waves per CU, 8 x 8 fragments per wave (moe_mfma_probe), "
                    "%.0f ms" % best[0],
            "tflops": round(tflops, 1), "frac_of_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
            "clock_ghz": round(best[1], 3)}


def vendor_gemm(torch, wl, counts, ours, reps=10):
    """The tile GEMMs' per-expert products run by torch.matmul (hipBLASLt on
    this system), for context beside the library's own stage times: GEMM 1
    as X_e [n_e, d] . [w1_e | w3_e] [d, 2f] (no SwiGLU, bf16 out) and GEMM 2
    as H_e [n_e, f] . w2_e [f, d] (bf16 out, where the library writes fp32),
    expert after expert, on random bf16 operands with the workload's
    per-expert row counts.  Each is timed with the weights in the layer's
    layout (n contiguous) and k contiguous (the layout of nn.Linear's
    weight).  Nothing in the layer calls it."""
    d, f = wl.d, wl.f
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    rows = [int(c) for c in counts if c > 0]
    out = {"what": "torch.matmul (hipBLASLt) bf16 on each expert's rows in turn: gemm1 = "
                   "x_e . [w1_e | w3_e] without the SwiGLU, gemm2 = h_e . w2_e; weights in the "
                   "layer's layout (n contiguous) and k contiguous; random operands",
           "rows_per_expert": rows}
    for gemm, kdim, ndim in (("gemm1", d, 2 * f), ("gemm2", f, d)):
        xs = [torch.randn(n, kdim, device="cuda", dtype=torch.bfloat16, generator=gen) for n in rows]
        ws = [torch.randn(kdim, ndim, device="cuda", dtype=torch.bfloat16, generator=gen)
              for _ in rows]
        flops = 2.0 * sum(rows) * kdim * ndim
        vendor = {}
        for layout in ("n_contiguous", "k_contiguous"):
            if layout == "k_contiguous":
                ws = [w.t().contiguous().t() for w in ws]  # same values, k fastest

            def run():
                for x, w in zip(xs, ws):
                    torch.matmul(x, w)

            for _ in range(3):
                run()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                run()
            b.record()
            torch.cuda.synchronize()
            vendor[layout] = round(a.elapsed_time(b) / reps, 5)
        del xs, ws
        torch.cuda.empty_cache()
        out[gemm] = {
            "ours_ms": ours[gemm], "ours_tflops": round(flops / (ours[gemm] * 1e-3) / 1e12, 1),
            "torch_matmul_ms": vendor,
            "torch_matmul_tflops": {kk: round(flops / (v * 1e-3) / 1e12, 1) for kk, v in vendor.items()},
            "vendor_ms_over_ours": {kk: round(v / ours[gemm], 4) for kk, v in vendor.items()},
        }
        log("[bench] vendor %s (%s rows): ours %.4f ms, torch.matmul %.4f ms (n-contiguous "
            "weights), %.4f ms (k-contiguous)" % (gemm, wl.name, ours[gemm], vendor["n_contiguous"],
                                                 vendor["k_contiguous"]))
    return out


POWER_COMMAND = "python3 bench.py --power-sample {secs}"


def power_sample(torch, binding, inputs, secs=10.0):
    """Board power while the layer runs: `amd-smi metric -p` polled in a
    thread (socket power, about four readings a second) during loops of the
    decode layer, the prefill layer and the MFMA probe, each about `secs`
    seconds after a short warm-up, with the power cap from `rocm-smi
    --showmaxpower`; written to profiles/board_power_decode_prefill_mfma.txt.
    A measurement aid only; the library does not read power."""
    import re
    import shutil
    import statistics
    import subprocess
    import threading

    smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    rsmi = shutil.which("rocm-smi") or "/opt/rocm/bin/rocm-smi"
    cap = None
    try:
        txt = subprocess.run([rsmi, "--showmaxpower"], capture_output=True, text=True, timeout=30).stdout
        m = re.search(r"Max Graphics Package Power \(W\):\s*([0-9.]+)", txt)
        cap = float(m.group(1)) if m else None
    except (OSError, subprocess.SubprocessError):
        pass
    samples = []
    on = threading.Event()
    on.set()

    def poll():
        while on.is_set():
            try:
                txt = subprocess.run([smi, "metric", "-p"], capture_output=True, text=True, timeout=10).stdout
            except (OSError, subprocess.SubprocessError):
                return
            m = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", txt)
            if m:
                samples.append((time.time(), float(m.group(1))))

    th = threading.Thread(target=poll, daemon=True)
    th.start()
    phases = []

    def phase(name, body):
        body(1.0)  # warm-up, not counted
        t0 = time.time()
        info = body(secs)
        phases.append((name, t0, time.time(), info))

    def idle(t):
        time.sleep(t)
        return ""

    def layer(which):
        wl = inputs.WORKLOADS[which]
        inp = inputs.workload_inputs(which, "cuda")
        out = torch.empty_like(inp["x"])

        def body(t):
            t0, n = time.time(), 0
            while time.time() - t0 < t:
                for _ in range(20):
                    binding.moe_ffn_forward(inp["x"], inp["w_router"], inp["w1"], inp["w3"], inp["w2"],
                                            wl.k, out=out)
                torch.cuda.synchronize()
                n += 20
            return "%.4f ms/step" % (1e3 * (time.time() - t0) / n)
        return body, inp

    phase("idle", idle)
    for which in ("decode", "prefill"):
        body, inp = layer(which)
        phase(which, body)
        del inp, body
        torch.cuda.empty_cache()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    ops = torch.randn(4 << 20, dtype=torch.float32, device="cuda").to(torch.bfloat16)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    clocks = torch.zeros(2 * cus, dtype=torch.int64, device="cuda")

    def mfma(t):
        t0 = time.time()
        while time.time() - t0 < t:
            binding.moe_mfma_probe(ops, 20000, cus, sink, clocks)
            torch.cuda.synchronize()
        ck = clocks.cpu().numpy().reshape(cus, 2).astype(float)
        return "clock %.3f GHz" % (ck[:, 0].sum() / ck[:, 1].sum() * 0.1)

    phase("mfma_probe", mfma)
    on.clear()
    th.join(timeout=15)
    out = os.path.join(ROOT, "profiles", "board_power_decode_prefill_mfma.txt")
    with open(out, "w") as fh:
        fh.write("# Board (socket) power while the layer runs: amd-smi metric -p polled during %.0f s loops "
                 "of the decode layer (T=32), the prefill layer (T=4096) and the MFMA probe\n" % secs)
        fh.write("# command: %s\n" % POWER_COMMAND.format(secs=int(secs)))
        fh.write("power_cap_w = %s  (rocm-smi --showmaxpower: Max Graphics Package Power)\n" % cap)
        for name, t0, t1, info in phases:
            w = [v for (t, v) in samples if t0 + 0.5 <= t <= t1]
            if not w:
                fh.write("%s: no readings\n" % name)
                continue
            fh.write("%s: median %.0f W, min %.0f, max %.0f, %d readings%s%s\n" % (
                name, statistics.median(w), min(w), max(w), len(w),
                (", %.3f of the cap" % (statistics.median(w) / cap)) if cap else "",
                ("; " + info) if info else ""))
    log("[bench] wrote", out)


def calibrate_copy(torch, nbytes=CALIBRATION_BYTES, reps=3):
    """Plain device-to-device copies of a known size (reference for the
    FETCH_SIZE / WRITE_SIZE counters)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[bench] calibration copy: %d x %d bytes" % (reps, nbytes))


def _counter_rows(run_dir):
    import csv
    path = os.path.join(run_dir, "run_counter_collection.csv")
    with open(path) as fh:
        return list(csv.DictReader(fh))


def summarize_counters(fetch_dir, write_dir, which="default"):
    """Turn two rocprofv3 --pmc runs of PMC_COMMAND (FETCH_SIZE, then
    WRITE_SIZE) into profiles/gemm1_swiglu_<workload>_traffic.txt for the
    decode and prefill workloads, or two runs of SKEWED_PMC_COMMAND
    (which="skewed") or STACK_PMC_COMMAND (which="stack") into that
    workload's: HBM bytes per launch of the w1/w3 kernel, each counter scaled
    by what it reads for the 1 GiB calibration copies run in the same
    process."""
    skewed = which == "skewed"
    stack = which == "stack"
    import re
    import statistics

    rows = {"FETCH_SIZE": _counter_rows(fetch_dir), "WRITE_SIZE": _counter_rows(write_dir)}
    factor, calib = {}, {}
    for name, rs in rows.items():
        vals = sorted(float(r["Counter_Value"]) for r in rs
                      if r["Counter_Name"] == name and "copyBuffer" in r["Kernel_Name"])
        if not vals:
            raise SystemExit("no calibration copy dispatches in the %s run" % name)
        # the calibration copies are the three largest copies of the run
        calib[name] = statistics.median(vals[-3:])
        factor[name] = CALIBRATION_BYTES / (calib[name] * 1024.0)
    written = []
    for wl, (src, pattern) in GEMM1_KERNEL.items():
        per = {}
        for name, rs in rows.items():
            vals = [float(r["Counter_Value"]) for r in rs
                    if r["Counter_Name"] == name and re.search(pattern, r["Kernel_Name"])]
            if vals:
                per[name] = vals
        if len(per) != 2 or (wl == "skewed") != skewed or (wl == "stack") != stack:
            continue
        if which == "default" and wl not in ("decode", "prefill"):
            continue
        fetch_kib = statistics.mean(per["FETCH_SIZE"])
        write_kib = statistics.mean(per["WRITE_SIZE"])
        hbm = fetch_kib * 1024.0 * factor["FETCH_SIZE"] + write_kib * 1024.0 * factor["WRITE_SIZE"]
        out = os.path.join(ROOT, "profiles", "gemm1_swiglu_%s_traffic.txt" % wl)
        with open(out, "w") as fh:
            fh.write("# HBM traffic of the w1/w3 grouped GEMM + SwiGLU kernel, %s workload\n" % wl)
            fh.write("# kernel: %s (source %s)\n" % (pattern, src))
            cmd = SKEWED_PMC_COMMAND if skewed else (STACK_PMC_COMMAND if stack else PMC_COMMAND)
            for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
                fh.write("# command (%s): %s\n" % (name, cmd.format(counter=name, out=d)))
            fh.write("# summarized by: python3 bench.py --summarize-counters %s %s%s\n"
                     % (fetch_dir, write_dir,
                        "" if which == "default" else " --counters-workload " + which))
            fh.write("# calibration: %d-byte device copy reads FETCH_SIZE %.1f KiB, WRITE_SIZE %.1f "
                     "KiB\n" % (CALIBRATION_BYTES, calib["FETCH_SIZE"], calib["WRITE_SIZE"]))
            fh.write("fetch_scale = %.4f\n" % factor["FETCH_SIZE"])
            fh.write("write_scale = %.4f\n" % factor["WRITE_SIZE"])
            fh.write("launches = %d\n" % len(per["FETCH_SIZE"]))
            fh.write("fetch_kib_per_launch = %.1f\n" % fetch_kib)
            fh.write("write_kib_per_launch = %.1f\n" % write_kib)
            fh.write("hbm_bytes_per_launch = %.0f\n" % hbm)
            fh.write("kernel_source_sha256_16 = %s\n" % source_digest(wl))
        written.append(out)
    for out in written:
        log("[bench] wrote", out)
    if not written:
        raise SystemExit("no w1/w3 kernel dispatches found")


def summarize_mfma(run_dir):
    """Turn one rocprofv3 --pmc run of MFMA_COMMAND into
    profiles/gemm1_swiglu_prefill_mfma.txt: per launch of the prefill w1/w3
    kernel its MFMA busy cycles (summed over all SIMDs), the bf16 MFMA work it
    issued (SQ_INSTS_VALU_MFMA_MOPS_BF16, units of 512 flops) against the
    algorithmic 4 T k d f, and the MFMA busy fraction over the dispatch's own
    duration at the nominal clock."""
    import re
    import statistics

    rows = _counter_rows(run_dir)
    pattern = GEMM1_KERNEL["prefill"][1]
    per = {}
    span = {}
    for r in rows:
        if not re.search(pattern, r["Kernel_Name"]):
            continue
        per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        span[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if len(per) < 4 or not span:
        raise SystemExit("no prefill w1/w3 dispatches with all counters in %s" % run_dir)
    avg = {k: statistics.mean(v) for k, v in per.items()}
    dur = statistics.mean(span.values())
    from sparse_mixture_experts_select_amd import inputs
    wl = inputs.WORKLOADS["prefill"]
    alg_flops = 4.0 * wl.T * wl.k * wl.d * wl.f
    issued_flops = avg["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512.0
    busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"]
    out = os.path.join(ROOT, "profiles", "gemm1_swiglu_prefill_mfma.txt")
    with open(out, "w") as fh:
        fh.write("# MFMA use of the w1/w3 grouped GEMM + SwiGLU kernel, prefill workload "
                 "(T=4096, d=4096, f=14336, E=8, k=2, bf16)\n")
        fh.write("# kernel: %s (source %s)\n" % (pattern, GEMM1_KERNEL["prefill"][0]))
        fh.write("# command: %s\n" % MFMA_COMMAND.format(out=run_dir))
        fh.write("# summarized by: python3 bench.py --summarize-mfma %s\n" % run_dir)
        fh.write("# counters per launch (averages over %d launches); SQ_VALU_MFMA_BUSY_CYCLES is "
                 "summed over all %d SIMDs (a 16x16x32 bf16 MFMA keeps its SIMD busy 16 cycles)\n"
                 % (len(span), SIMDS))
        for k in sorted(avg):
            fh.write("%s = %.0f\n" % (k, avg[k]))
        fh.write("dispatch_seconds = %.6e\n" % dur)
        fh.write("algorithmic_flops = %.6e\n" % alg_flops)
        fh.write("issued_mfma_flops = %.6e\n" % issued_flops)
        fh.write("issued_over_algorithmic = %.4f  (rows of partial tiles computed and not stored)\n"
                 % (issued_flops / alg_flops))
        fh.write("mfma_busy_cycles_per_simd = %.0f\n" % (busy / SIMDS))
        fh.write("mfma_busy_fraction_at_2.4GHz = %.4f  (busy cycles / (SIMDs x duration x 2.4 GHz))\n"
                 % (busy / (SIMDS * dur * NOMINAL_CLOCK_HZ)))
        # GRBM_GUI_ACTIVE counts the cycles the GPU is busy, summed over its 8
        # XCDs, at the clock it actually runs (cross-checked against a kernel
        # probe of s_memtime against the 100 MHz real-time counter)
        clock = avg["GRBM_GUI_ACTIVE"] / 8 / dur
        fh.write("clock_ghz_from_grbm = %.3f  (GRBM_GUI_ACTIVE / 8 XCDs / duration)\n" % (clock / 1e9))
        fh.write("mfma_busy_fraction_at_that_clock = %.4f\n" % (busy / (SIMDS * dur * clock)))
        fh.write("achieved_tflops_in_dispatch = %.1f\n" % (alg_flops / dur / 1e12))
        fh.write("bf16_peak_at_that_clock_tflops = %.1f\n" % (SIMDS * 1024 * clock / 1e12))
    log("[bench] wrote", out)


def summarize_stalls(run_dirs):
    """Turn the four rocprofv3 --pmc passes of STALL_COMMAND (STALL_PASSES in
    order) into profiles/tile_gemm_prefill_wave_states.txt: for the prefill
    w1/w3 kernel and the w2 kernel, the counters per launch and where the
    waves' cycles go.  SQ_WAVE_CYCLES, SQ_WAIT_ANY, SQ_WAIT_INST_ANY and
    SQ_ACTIVE_INST_ANY count in units of 4 cycles (4 x SQ_WAVE_CYCLES comes
    to 0.95 of SIMDs x duration x clock for these kernels, which hold one
    wave per SIMD); SQ_VALU_MFMA_BUSY_CYCLES counts cycles (16 per
    16x16x32 bf16 MFMA)."""
    import re
    import statistics

    kernels = (("w1/w3 grouped GEMM + SwiGLU", GEMM1_KERNEL["prefill"][1]),
               ("w2 grouped GEMM", r"tile_gemm_kernel(<false, (true|false)>|ILb0ELb[01]E)"))
    per = {name: {} for name, _ in kernels}
    span = {name: {} for name, _ in kernels}
    for d in run_dirs:
        for r in _counter_rows(d):
            for name, pattern in kernels:
                if re.search(pattern, r["Kernel_Name"]):
                    key = (d, r["Dispatch_Id"])
                    per[name].setdefault(r["Counter_Name"], {}).setdefault(key, 0.0)
                    per[name][r["Counter_Name"]][key] += float(r["Counter_Value"])
                    span[name][key] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    out = os.path.join(ROOT, "profiles", "tile_gemm_prefill_wave_states.txt")
    with open(out, "w") as fh:
        fh.write("# Wave states of the 256x256 tile GEMMs, prefill workload (T=4096, d=4096, f=14336, "
                 "E=8, k=2, bf16)\n")
        fh.write("# kernels: %s (source %s), and GEMM 2\n" % (kernels[0][1], GEMM1_KERNEL["prefill"][0]))
        for i, counters in enumerate(STALL_PASSES):
            fh.write("# command (pass %d): %s\n" % (i + 1, STALL_COMMAND.format(
                counters=counters, out=run_dirs[i] if i < len(run_dirs) else "?")))
        fh.write("# summarized by: python3 bench.py --summarize-stalls %s\n" % " ".join(run_dirs))
        fh.write("# counters per launch, averaged over the launches of each pass; SQ_WAVE_CYCLES, "
                 "SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_ACTIVE_INST_ANY in units of 4 cycles\n")
        fh.write("kernel_source_sha256_16 = %s\n" % source_digest("prefill"))
        for name, _ in kernels:
            c = {k: statistics.mean(v.values()) for k, v in per[name].items()}
            if "SQ_WAVE_CYCLES" not in c or "SQ_INSTS_MFMA" not in c:
                raise SystemExit("missing counters for %s in %s" % (name, run_dirs))
            dur = statistics.mean(t for t in span[name].values())
            fh.write("\n[%s]\n" % name)
            for k in sorted(c):
                fh.write("%s = %.4g\n" % (k, c[k]))
            wave = 4.0 * c["SQ_WAVE_CYCLES"]
            clock = c["GRBM_GUI_ACTIVE"] / 8 / dur
            waves = c["SQ_WAVES"]
            fh.write("dispatch_seconds = %.4e\n" % dur)
            fh.write("clock_ghz_from_grbm = %.3f\n" % (clock / 1e9))
            fh.write("wave_residency = %.3f  (4 SQ_WAVE_CYCLES / (SIMDs x duration x clock))\n"
                     % (wave / (SIMDS * dur * clock)))
            fh.write("mfma_busy_of_wave_cycles = %.3f\n" % (c["SQ_VALU_MFMA_BUSY_CYCLES"] / wave))
            fh.write("waiting_on_waitcnt_or_barrier = %.3f  (SQ_WAIT_ANY / SQ_WAVE_CYCLES)\n"
                     % (c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]))
            fh.write("ready_but_not_issued = %.3f  (SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES: mostly the "
                     "next MFMA waiting for the matrix core)\n" % (c["SQ_WAIT_INST_ANY"] / c["SQ_WAVE_CYCLES"]))
            fh.write("issuing = %.3f  (SQ_ACTIVE_INST_ANY / SQ_WAVE_CYCLES)\n"
                     % (c["SQ_ACTIVE_INST_ANY"] / c["SQ_WAVE_CYCLES"]))
            fh.write("lds_bank_conflict_cycles_per_lds_instruction = %.4f\n"
                     % (c["SQ_LDS_BANK_CONFLICT"] / c["SQ_INSTS_LDS"]))
            fh.write("per wave: mfma %.0f, valu (SQ_INSTS_VALU, MFMAs included) %.0f, salu %.0f, lds %.0f, "
                     "vmem %.0f instructions\n"
                     % (c["SQ_INSTS_MFMA"] / waves, c["SQ_INSTS_VALU"] / waves,
                        c["SQ_INSTS_SALU"] / waves, c["SQ_INSTS_LDS"] / waves, c["SQ_INSTS_VMEM"] / waves))
    log("[bench] wrote", out)


def _short_kernel_name(name):
    """Readable kernel name: the library's mangled names (plain function
    templates over bool / int / bf16 / float) are decoded by hand."""
    import re
    m = re.match(r"_ZN3moe12_GLOBAL__N_1(\d+)", name)
    if m:
        n = int(m.group(1))
        base = name[m.end():m.end() + n]
        rest = name[m.end() + n:]
        if rest.startswith("I"):
            args = []
            for tok in re.finditer(r"Lb([01])E|Li(-?\d+)E|DF16b|f", rest[1:rest.index("EE") + 1]):
                if tok.group(1) is not None:
                    args.append("true" if tok.group(1) == "1" else "false")
                elif tok.group(2) is not None:
                    args.append(tok.group(2))
                else:
                    args.append("bf16" if tok.group(0) == "DF16b" else "float")
            base += "<%s>" % ", ".join(args)
        return base
    name = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    depth = 0
    for i, ch in enumerate(name):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0:
            return name[:i]
    return name


def summarize_trace(trace_dir):
    """Condense the --kernel-trace output of TRACE_COMMAND into
    profiles/moe_layer_decode_prefill_stack_kernel_stats.txt: per kernel and grid
    size (which tells the workloads' launches apart) the number of
    calls and the average / min / max duration."""
    import csv
    import statistics
    with open(os.path.join(trace_dir, "run_kernel_trace.csv")) as fh:
        rows = list(csv.DictReader(fh))
    groups = {}
    phase = None  # the router launch that opened the current layer call
    garbled = False
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    rows = [r for r in rows if "moe" in r["Kernel_Name"] or "copyBuffer" in r["Kernel_Name"]]
    for i, r in enumerate(rows):
        name = _short_kernel_name(r["Kernel_Name"])
        if "_Accum" in name:
            # rocprofv3 prints combine_kernel<bf16, true> (the K-slice form,
            # the only combine instantiation with a bool true that the
            # benchmark runs) with this garbled template list
            name, garbled = "combine_kernel<bf16, true>", True
        grid = int(r["Grid_Size_X"])
        if name.startswith("router_"):
            # a router launch opens a layer call; the launch after it (the
            # grouping, sized by T*k) tells workloads apart whose routers
            # share a grid
            nxt = rows[i + 1] if i + 1 < len(rows) else r
            phase = (name, grid, nxt["Kernel_Name"], int(nxt["Grid_Size_X"]))
        key = (phase, name, grid)
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        g = groups.setdefault(key, {"d": [], "first": int(r["Dispatch_Id"]), "row": r})
        g["d"].append(dur)
    out = os.path.join(ROOT, "profiles", "moe_layer_decode_prefill_stack_kernel_stats.txt")
    with open(out, "w") as fh:
        fh.write("# rocprofv3 kernel trace of the benchmark: decode (T=32), prefill (T=4096), "
                 "skewed routing (T=16384), then the 32-block stack (T=2048; one layer call per "
                 "block, RMSNorm formed by the router); d=4096 f=14336 E=8 k=2 bf16\n")
        fh.write("# command: %s\n" % TRACE_COMMAND.format(out=trace_dir))
        fh.write("# summarized by: python3 bench.py --summarize-trace %s\n" % trace_dir)
        fh.write("# calls = warm-up + one routing probe call + timed steps; durations in us; "
                 "grid in work-items; torch's input generation kernels left out; rows are grouped "
                 "per workload (the router launch that opens each layer call)\n")
        if garbled:
            fh.write("# combine_kernel<bf16, true>: rocprofv3 printed this instantiation's name as "
                     "'combine_kernel<bool _Accum, bool, E>'\n")
        fh.write("%-44s %9s %6s %10s %10s %10s %5s %5s %6s %7s\n" % (
            "kernel", "grid", "calls", "avg_us", "min_us", "max_us", "vgpr", "agpr", "lds",
            "scratch"))
        for (_, name, grid), g in sorted(groups.items(), key=lambda kv: kv[1]["first"]):
            r = g["row"]
            fh.write("%-44s %9d %6d %10.2f %10.2f %10.2f %5s %5s %6s %7s\n" % (
                name[:44], grid, len(g["d"]), statistics.mean(g["d"]), min(g["d"]), max(g["d"]),
                r["VGPR_Count"], r["Accum_VGPR_Count"], r["LDS_Block_Size"],
                r.get("Scratch_Size", "?")))
    log("[bench] wrote", out)


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "skewed"])
    ap.add_argument("--secondary", default="prefill", choices=["prefill", "decode", "skewed", "none"])
    ap.add_argument("--skewed", default="on", choices=["on", "off"],
                    help="also run the skewed-routing workload (T=16384, biased router)")
    ap.add_argument("--stack", default="on", choices=["on", "off"],
                    help="also time the 32-block stack (90 GB of weights resident)")
    ap.add_argument("--sweep", default="on", choices=["on", "off"],
                    help="also time the layer over T = 1 .. 16384 (prefill weights)")
    ap.add_argument("--vendor", default="on", choices=["on", "off"],
                    help="time torch.matmul (hipBLASLt) on the prefill workload's per-expert "
                         "GEMM shapes beside the library's GEMM stages")
    ap.add_argument("--sweep-steps", type=int, default=5,
                    help="timed steps per batch size in the sweep")
    ap.add_argument("--cpu-full", nargs="+", default=["tiny", "prefill"],
                    choices=["tiny", "decode", "prefill", "none"],
                    help="workloads the oracle is also timed on in full")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--counters-workload", default="default", choices=["default", "skewed", "stack"],
                    help="with --summarize-counters: the runs are of PMC_COMMAND (default), "
                         "SKEWED_PMC_COMMAND or STACK_PMC_COMMAND")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR")
    ap.add_argument("--power-sample", type=float, metavar="SECONDS",
                    help="only sample board power during decode, prefill and MFMA-probe loops of "
                         "this length and write the profile")
    ap.add_argument("--summarize-stalls", nargs=4, metavar="PMC_DIR",
                    help="the four counter passes of STALL_COMMAND, in STALL_PASSES order")
    args = ap.parse_args()

    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, which=args.counters_workload)
        return
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return
    if args.summarize_stalls:
        summarize_stalls(args.summarize_stalls)
        return

    if args.gpus != 1:
        print("bench.py measures one GPU only: this layer is benchmarked on a single MI355X "
              "(--gpus 1); runs on %d GPUs are not supported." % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_mixture_experts_select_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)

    if args.power_sample:
        power_sample(torch, binding, inputs, args.power_sample)
        return

    prim = run_workload(args.workload, args.steps, args.warmup, binding, inputs, torch)
    bound = "hbm" if args.workload == "decode" else "mfma"
    if bound == "hbm":
        probe = read_probe(torch, binding, [prim["inp"][n] for n in ("w1", "w3", "w2")])
    wl = prim["wl"]
    rec = {
        "metric": METRIC,
        "value": round(prim["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(prim["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "%s (T=%d, d=%d, f=%d, E=%d, k=%d)" % (wl.name, wl.T, wl.d, wl.f, wl.E, wl.k),
                   "T": wl.T, "d": wl.d, "f": wl.f, "E": wl.E, "k": wl.k, "parallelism": "single GPU"},
        "roofline": roofline(prim, bound),
        "layer": {"tflops_active": round(prim["layer_tflops"], 2),
                  "mfma_frac": round(prim["layer_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                  "hbm_gbs": round(prim["layer_gbs"], 1),
                  "hbm_frac": round(prim["layer_gbs"] / HBM_PEAK_GBS, 4),
                  "design_bytes_per_layer": design_traffic(wl, "gather_rows" in prim["stage_ms"])},
        "stages_ms": prim["stage_ms"],
        "stages_roofline": prim["stage_roofline"],
        "step_ms": prim["step_ms"],
        "device": device_facts(torch),
        "note": ("each step streams the expert weights from HBM: one layer's 2.82 GB exceeds the "
                 "256 MiB MALL, so no cache flush is needed between steps"),
    }
    overrides = {n: os.environ[n] for n in ("MOE_FFN_STREAM_SPLITS", "MOE_FFN_STREAM_K_WAVES")
                 if os.environ.get(n)}
    if overrides:
        rec["plan_overrides"] = overrides
    side_counts = {}

    def side_workload(name):
        # free the primary inputs while another workload runs
        prim_inp = prim.pop("inp")
        torch.cuda.empty_cache()
        res = run_workload(name, args.steps, args.warmup, binding, inputs, torch)
        res.pop("inp")
        torch.cuda.empty_cache()
        prim["inp"] = prim_inp
        side_counts[name] = res["counts"]
        out = {
            "workload": name, "value": round(res["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_step": round(res["ms_per_step"], 5),
            "roofline": roofline(res, "hbm" if name == "decode" else "mfma"),
            "layer": {"tflops_active": round(res["layer_tflops"], 2),
                      "mfma_frac": round(res["layer_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                      "hbm_gbs": round(res["layer_gbs"], 1),
                      "design_bytes_per_layer": design_traffic(inputs.WORKLOADS[name],
                                                               "gather_rows" in res["stage_ms"])},
            "stages_ms": res["stage_ms"],
            "stages_roofline": res["stage_roofline"],
            "step_ms": res["step_ms"],
        }
        if name == "skewed":
            c = res["counts"]
            out["expert_share"] = [round(v / sum(c), 4) for v in c]
        return out

    if args.secondary != "none" and args.secondary != args.workload:
        rec["secondary"] = side_workload(args.secondary)
    if args.skewed == "on" and args.workload != "skewed" and args.secondary != "skewed":
        rec["skewed"] = side_workload("skewed")
    if args.vendor == "on" and "prefill" in (args.workload, args.secondary):
        pre = rec["stages_ms"] if args.workload == "prefill" else rec["secondary"]["stages_ms"]
        counts = prim["counts"] if args.workload == "prefill" else side_counts["prefill"]
        prim_inp = prim.pop("inp")
        torch.cuda.empty_cache()
        try:
            rec["vendor_gemm"] = vendor_gemm(torch, inputs.WORKLOADS["prefill"], counts,
                                             {"gemm1": pre["gemm1_swiglu"], "gemm2": pre["gemm2"]})
        except Exception as exc:  # a comparison only: its failure must not cost the line
            rec["vendor_gemm"] = {"error": "%s: %s" % (type(exc).__name__, exc)}
            log("[bench] vendor GEMM comparison failed:", exc)
        torch.cuda.empty_cache()
        prim["inp"] = prim_inp
    if args.sweep == "on":
        prim_inp = prim.pop("inp")
        del prim_inp
        torch.cuda.empty_cache()
        rec["sweep"] = run_sweep(args.sweep_steps, min(args.warmup, 2), binding, inputs, torch)
        torch.cuda.empty_cache()
        prim["inp"] = inputs.workload_inputs(args.workload, "cuda")
    if args.stack == "on":
        prim_inp = prim.pop("inp")
        del prim_inp
        torch.cuda.empty_cache()
        rec["stack"] = run_stack(max(2, args.steps // 4), 1, binding, inputs, torch)
        torch.cuda.empty_cache()
        prim["inp"] = inputs.workload_inputs(args.workload, "cuda")
    if args.calibrate_copy:
        calibrate_copy(torch)
    rec["mfma_probe"] = mfma_probe(torch, binding)
    for key in ("secondary", "skewed", "stack"):
        rl = rec.get(key, {}).get("roofline")
        if rl and rl["bound"] == "mfma":
            rl["frac_of_mfma_probe"] = round(rl["achieved"] / rec["mfma_probe"]["tflops"], 4)
    if bound == "mfma":
        rec["roofline"]["frac_of_mfma_probe"] = round(
            rec["roofline"]["achieved"] / rec["mfma_probe"]["tflops"], 4)
    if bound == "hbm":
        gbs, nbytes, grids = probe
        rec["read_probe"] = {
            "what": "streaming read of the timed layer's own w1, w3 and w2 (%d bytes), nontemporal "
                    "16-byte loads, fastest grid per buffer %s workgroups of 256 (moe_hbm_read_probe)"
                    % (nbytes, "/".join(str(g) for g in grids)),
            "gbs": round(gbs, 1),
            "gemm1_frac_of_probe": round(rec["roofline"]["achieved"] / gbs, 4),
            "layer_frac_of_probe": round(prim["layer_gbs"] / gbs, 4),
        }
    if args.no_cpu_baseline:
        rec["cpu_baseline"] = None
    else:
        rec["cpu_baseline"] = cpu_baseline(prim, args.cpu_seconds, inputs, torch,
                                           full=tuple(w for w in args.cpu_full if w != "none"))
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
