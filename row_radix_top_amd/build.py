"""Build the HIP library ``row_radix_top_amd/lib/libtopk_ragged.so`` for gfx950.

``python -m row_radix_top_amd.build`` (or ``__graft_entry__.build()``) always
recompiles.  The library is built in-tree so it travels with the source tree.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libtopk_ragged.so")
SOURCES = [os.path.join(CSRC, "topk_kernels.hip"), os.path.join(CSRC, "topk_host.cpp"),
           os.path.join(CSRC, "topk_noalloc.hip")]

HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # The streaming compare relies on IEEE subnormal handling.
    "-fno-gpu-flush-denormals-to-zero",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIP_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
