"""The plan overrides MOE_FFN_STREAM_SPLITS and MOE_FFN_STREAM_K_WAVES
(read once per process) change the streamed path's kernel shapes, not its
results: a child process per setting checks every element of small shapes
against the oracle, and its workspace sizes show the slice count it ran."""
import os
import re
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
CHILD = os.path.join(HERE, "override_parity_child.py")


@pytest.mark.parametrize("splits,k_waves", [(3, 2), (2, 1)])
def test_overrides_keep_parity(splits, k_waves):
    from sparse_mixture_experts_select_amd import binding
    from override_parity_child import CASES
    env = dict(os.environ)
    env["MOE_FFN_STREAM_SPLITS"] = str(splits)
    env["MOE_FFN_STREAM_K_WAVES"] = str(k_waves)
    print("\n[case] child with MOE_FFN_STREAM_SPLITS=%d MOE_FFN_STREAM_K_WAVES=%d" % (splits, k_waves),
          flush=True)
    out = subprocess.run([sys.executable, "-u", CHILD], env=env, capture_output=True, text=True,
                         timeout=240)
    print(out.stdout[-3000:], out.stderr[-3000:])
    assert out.returncode == 0
    ws = [int(m) for m in re.findall(r"^ok T=\d+ workspace (\d+)", out.stdout, re.M)]
    assert len(ws) == len(CASES)
    for (T, d, f, E, k), child_ws in zip(CASES, ws):
        own = binding.moe_ffn_workspace_bytes(T, d, f, E, k)  # this process: the plan's choice
        own_splits = None
        # the y slices are the only part of the workspace that depends on the
        # slice count: R x d fp32 each
        R = T * k
        for s in range(1, 17):
            if own - (s - splits) * R * d * 4 == child_ws:
                own_splits = s
        assert own_splits is not None and own_splits != splits, (own, child_ws)
