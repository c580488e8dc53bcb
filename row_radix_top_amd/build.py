"""Build the HIP library ``row_radix_top_amd/lib/libtopk_ragged.so`` for gfx950.

``python -m row_radix_top_amd.build`` (or ``__graft_entry__.build()``) always
recompiles.  The kernel instances are spread over several translation units
that compile in parallel (objects under ``_build/``); the library is linked
in-tree so it travels with the source tree.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libtopk_ragged.so")
OBJDIR = os.path.join(PKG, "_build")


def sources() -> list[str]:
    hips = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    return [os.path.join(CSRC, "topk_host.cpp"), *hips]


HIP_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
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


def _compile(src: str, extra: list[str], verbose: bool) -> tuple[str, float]:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIP_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {os.path.basename(src)} failed:\n{err}")
    if err.strip() and verbose:
        print(err, flush=True)
    return obj, time.time() - t0


def build(verbose: bool = False, extra_flags: list[str] | None = None, jobs: int | None = None) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    os.makedirs(OBJDIR, exist_ok=True)
    extra = list(extra_flags or [])
    srcs = sources()
    jobs = jobs or max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "0") or 0) or (os.cpu_count() or 1), 16))
    t0 = time.time()
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        futs = {ex.submit(_compile, s, extra, verbose): s for s in srcs}
        objs = {}
        for f in cf.as_completed(futs):
            obj, dt = f.result()
            objs[futs[f]] = obj
            if verbose:
                print(f"  {os.path.basename(futs[f])}: {dt:.1f} s", flush=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", "--offload-arch=gfx950", *[objs[s] for s in srcs], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f} s ({jobs} jobs)", flush=True)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-q" not in sys.argv))
