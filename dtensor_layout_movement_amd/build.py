"""Build the reshard library (``libreshard.so``) in-tree for gfx950.

Run ``python -m dtensor_layout_movement_amd.build`` (or call ``build()``).  The
library is always rebuilt: hipcc cross-compiles the gfx950 code object on a
machine without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(REPO_DIR, "include")
LIB_PATH = os.path.join(PKG_DIR, "libreshard.so")
SOURCES = [os.path.join(CSRC, "plan.cpp"), os.path.join(CSRC, "kernel.hip"), os.path.join(CSRC, "reshard.hip")]

# Packed-fp32 instructions are kept out of every HIP object; the library does no
# floating point, so this costs nothing.
HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    "--offload-arch=gfx950",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the reshard library needs ROCm's hipcc")


def build(verbose: bool = False) -> str:
    """Compile plan.cpp + kernel.hip + reshard.hip into libreshard.so; return its path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, "-shared", "-I", INCLUDE, "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; drop that line
    noise = ("packed-fp32-ops", "warning: feature flag")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
