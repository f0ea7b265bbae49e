"""Build libmoe_ffn.so for gfx950 with hipcc (in-tree, under ``_build/``).

Usage: ``python -m sparse_mixture_experts_select_amd.build``.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_NAME = "libmoe_ffn.so"
LIB_PATH = os.path.join(BUILD_DIR, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["router.hip", "route_permute.hip", "gemm_bf16.hip", "gemm_stream.hip", "gemm_tile.hip", "gemm_tile_nt.hip", "gemm_f32.hip", "combine.hip", "probe.hip", "api.hip"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags(extra=()) -> list[str]:
    return [
        "--offload-arch=" + ARCH,
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-result",
        # Leave packed-fp32 instructions out of the generated code.
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
        *extra,
    ]


def _compile(src: str, obj: str, extra) -> None:
    cmd = [hipcc(), "-c", os.path.join(CSRC, src), "-o", obj, *compile_flags(extra)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, res.stdout, res.stderr))
    noise = [ln for ln in res.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if noise:
        sys.stderr.write("\n".join(noise) + "\n")


def build(extra=(), jobs: int = 8) -> str:
    """Compile every HIP source and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o") for s in SOURCES]
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = [ex.submit(_compile, s, o, tuple(extra)) for s, o in zip(SOURCES, objs)]
        for fu in futs:
            fu.result()
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (res.stdout, res.stderr))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
