"""Build the gfx950 shared library ``libbpt.so`` in-tree with hipcc.

Usage: ``python -m memory_efficient_long_amd.build`` (also called by
``__graft_entry__.build()``). Always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_PATH = os.path.join(PKG_DIR, "libbpt.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-munsafe-fp-atomics",
    # Packed fp32 VALU forms are disabled (hipcc still vectorises scalar code).
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]


# roctx ranges (only emitted when BPT_ROCTX=1; see the host code).
LINK_FLAGS = ["-lrocprofiler-sdk-roctx"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm toolchain required to build libbpt.so)")


def build(verbose: bool = False, out: str = LIB_PATH, csrc: str = CSRC, defines=()) -> str:
    src = os.path.join(csrc, "bpt_layer.hip")
    tmp = out + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *[f"-D{d}" for d in defines], "-I", os.path.join(REPO, "include"),
           src, "-o", tmp, *LINK_FLAGS]
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr[-6000:]}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
