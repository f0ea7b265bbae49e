"""Run in a child process by tests/test_gpu_overrides.py with the plan
overrides set in its environment (they are read once per process): parity of
the few-rows-per-expert path with the oracle on every element of small
shapes, and the workspace size each shape then needs.  Prints one line per
case and exits non-zero on any mismatch."""
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
for p in (os.path.dirname(HERE), HERE):
    if p not in sys.path:
        sys.path.insert(0, p)

import torch  # noqa: E402

import parity as PT  # noqa: E402
from sparse_mixture_experts_select_amd import binding, inputs  # noqa: E402

CASES = [(8, 256, 1024, 8, 2), (3, 256, 2048, 8, 2), (30, 192, 640, 8, 2)]


def main():
    for T, d, f, E, k in CASES:
        print("[case] T=%d d=%d f=%d E=%d k=%d under %s" % (
            T, d, f, E, k, {n: os.environ.get(n) for n in ("MOE_FFN_STREAM_SPLITS",
                                                           "MOE_FFN_STREAM_K_WAVES")}), flush=True)
        inp = inputs.make_weights(d, f, E, torch.bfloat16, "cuda", T + d, "override")
        inp["x"] = inputs.make_x(T, d, torch.bfloat16, "cuda", "rms", T + d, "override")
        inp["bias"] = None
        r = PT.full_check(inp, k)
        ws = binding.moe_ffn_workspace_bytes(T, d, f, E, k)
        print("ok T=%d workspace %d err %s" % (T, ws, (r["err_out"], r["err_h"], r["err_y"])), flush=True)


if __name__ == "__main__":
    main()
