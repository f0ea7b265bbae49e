"""Benchmark of the MoE feed-forward layer on one MI355X.

Prints ONE JSON line on stdout.  A step is one full layer call
(router + top-k/softmax, grouping, both grouped GEMMs, combine) over one batch
of synthetic inputs that are already resident in HBM.  The primary workload is
the T=32 decode batch at Mixtral shapes (d=4096, f=14336, E=8, k=2, bf16),
which is HBM-bound; the T=4096 prefill batch (MFMA-bound) is reported beside
it under "secondary".

Live timing: the K timed steps are bracketed by torch.cuda.synchronize();
inside them the library records HIP events at every stage boundary on the
launch stream (moe_ffn_profile_begin/end), which gives the average duration
of each kernel over the timed region.  The roofline entry is for the dominant
kernel (the w1/w3 grouped GEMM with the SwiGLU epilogue).

The CPU baseline times the fp64 oracle on the host on a bounded sample of the
same workload.
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
GEMM1_SOURCE = os.path.join(ROOT, "sparse_mixture_experts_select_amd", "csrc", "gemm_bf16.hip")


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


def source_digest(path):
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


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
    if vals.get("kernel_source_sha256_16") != source_digest(GEMM1_SOURCE):
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
    binding.moe_ffn_profile_begin(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    stage_ms, calls = binding.moe_ffn_profile_end()
    assert calls == steps, (calls, steps)
    stage_avg = {kk: v / calls for kk, v in stage_ms.items()}
    ms_per_step = 1e3 * elapsed / steps

    g_bytes, g_flops = gemm1_algorithmic(wl, counts_h)
    g_ms = stage_avg["gemm1_swiglu"]
    l_flops, l_bytes = layer_algorithmic(wl, counts_h)
    res = {
        "workload": name,
        "wl": wl,
        "inp": inp,
        "ms_per_step": ms_per_step,
        "tokens_per_s": wl.T / (ms_per_step * 1e-3),
        "stage_ms": {kk: round(v, 5) for kk, v in stage_avg.items()},
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


def cpu_baseline(res, seconds, inputs):
    """The fp64 oracle on the host cores on a bounded sample of the workload."""
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
    tok_s = reps * n_tok / el
    return {"value": round(tok_s, 3), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "%s workload, tokens 0..%d (full layer per token in fp64), %d passes, %.1f s"
                      % (wl.name, n_tok - 1, reps, el)}


def calibrate_copy(torch, nbytes=1 << 30, reps=3):
    """Plain device-to-device copies of a known size (reference for the
    FETCH_SIZE / WRITE_SIZE counters)."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("[bench] calibration copy: %d x %d bytes" % (reps, nbytes))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "skewed"])
    ap.add_argument("--secondary", default="prefill", choices=["prefill", "decode", "skewed", "none"])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true")
    args = ap.parse_args()

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

    prim = run_workload(args.workload, args.steps, args.warmup, binding, inputs, torch)
    bound = "hbm" if args.workload == "decode" else "mfma"
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
                  "hbm_frac": round(prim["layer_gbs"] / HBM_PEAK_GBS, 4)},
        "stages_ms": prim["stage_ms"],
    }
    if args.secondary != "none" and args.secondary != args.workload:
        # free the primary inputs before the secondary workload
        prim_inp = prim.pop("inp")
        sec = run_workload(args.secondary, args.steps, args.warmup, binding, inputs, torch)
        sbound = "hbm" if args.secondary == "decode" else "mfma"
        sec.pop("inp")
        rec["secondary"] = {
            "workload": args.secondary, "value": round(sec["tokens_per_s"], 1), "unit": "tokens/s",
            "ms_per_step": round(sec["ms_per_step"], 5),
            "roofline": roofline(sec, sbound),
            "layer": {"tflops_active": round(sec["layer_tflops"], 2),
                      "mfma_frac": round(sec["layer_tflops"] / MFMA_BF16_PEAK_TFLOPS, 4),
                      "hbm_gbs": round(sec["layer_gbs"], 1)},
            "stages_ms": sec["stage_ms"],
        }
        prim["inp"] = prim_inp
    if args.calibrate_copy:
        calibrate_copy(torch)
    if args.no_cpu_baseline:
        rec["cpu_baseline"] = None
    else:
        rec["cpu_baseline"] = cpu_baseline(prim, args.cpu_seconds, inputs)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
