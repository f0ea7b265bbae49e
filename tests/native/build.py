"""Build the native C check of the library's C ABI (tests/native/moe_abi_check.c).

Test infrastructure: gcc, linked against the HIP runtime, libmoe_ffn.so and
the CPU oracle (both must be built first).  Called by __graft_entry__.build();
tests/test_gpu_zz_native.py runs the result on a GPU.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "moe_abi_check.c")
BUILD_DIR = os.path.join(HERE, "_build")
EXE = os.path.join(BUILD_DIR, "moe_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    # library search paths relative to the executable, so the tree can move
    rpath = ":".join(["$ORIGIN/../../../sparse_mixture_experts_select_amd/_build",
                      "$ORIGIN/../../../oracle/_build", os.path.join(ROCM, "lib")])
    tmp = EXE + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "oracle"), SRC, "-o", tmp,
           "-L", os.path.join(ROOT, "sparse_mixture_experts_select_amd", "_build"), "-lmoe_ffn",
           "-L", os.path.join(ROOT, "oracle", "_build"), "-lmoe_oracle",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", "-lm", "-Wl,-rpath," + rpath]
    subprocess.run(cmd, check=True)
    os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build())
