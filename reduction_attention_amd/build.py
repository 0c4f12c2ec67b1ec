"""Build libattn.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["api.cpp", "decode.hip", "prefill.hip", "bsr_rows.hip", "mla.hip", "scratch.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # the kernels never produce NaN from finite inputs and handle -inf
    # explicitly: let max/min skip NaN canonicalisation
    "-fno-honor-nans",
    # packed fp32 VALU forms stay off: the compiler may not emit them
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    srcs = []
    for s in SOURCES:
        path = os.path.join(CSRC, s)
        # hipcc treats .cpp as host C++; compile every source as HIP
        srcs += ["-x", "hip", path]
    tmp = LIB + ".tmp"
    cmd = [hipcc] + HIPCC_FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed building libattn.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
