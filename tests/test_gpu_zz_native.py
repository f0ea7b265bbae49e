"""The layer driven from a plain C program through the C ABI (no Python in
the loop), checked against the CPU oracle inside that program: the tile and
streamed GEMM paths, E = 16 / k = 4, fp32, and two argument checks."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "native", "_build", "moe_abi_check")


def test_native_c_program_matches_oracle():
    print("\n[case] native C check of the C ABI", flush=True)
    if not os.path.exists(EXE):
        pytest.skip("%s is not built (run __graft_entry__.build())" % EXE)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=240)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "PASSED" in res.stdout
