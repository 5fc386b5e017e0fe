"""Build the gfx950 shared library ``libexact_row_top.so`` in-tree with hipcc.

Run as ``python -m exact_row_top_amd.build`` (or through
``__graft_entry__.build()``).  The build always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libexact_row_top.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["gvr_kernels.hip", "blockskip.hip", "epilogue.hip", "state.hip", "calib.hip",
           "topk_abi.cpp"]

# -ffp-contract=off: the histogram bin is one definition evaluated in several
#   passes; no pass may fuse it differently.
# -fno-gpu-flush-denormals-to-zero: fp32 denormals are ordinary scores.
# -target-feature -packed-fp32-ops: no packed fp32 VALU forms.
HIP_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, save_temps: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc, *HIP_FLAGS, "-I", INCLUDE, "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if save_temps and src.endswith(".hip"):
            cmd += ["-save-temps=obj"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.check_call(cmd, cwd=BUILD_DIR)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd, cwd=BUILD_DIR)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, save_temps="--save-temps" in sys.argv)
    print(LIB)
