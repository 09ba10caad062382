"""Build the gfx950 HIP library libk3moe.so in-tree with hipcc.

Usage: python -m mxfp4_routed_expert_softmax_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SO = os.path.join(HERE, "libk3moe.so")
SOURCES = ["api.hip", "route.hip", "gemv.hip", "mx.hip", "slices.hip", "cache.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Werror",
    "-Wno-unused-result",
    # packed fp32 VALU ops stay off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # keep fp32 denormals (the MX decode and quantiser rely on exact values)
    "-fno-gpu-flush-denormals-to-zero",
    "-fno-fast-math",
    # a missing definition must fail the link, not the first dlopen
    "-Wl,-z,defs",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err)
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
