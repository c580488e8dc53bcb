"""Build the CPU oracle library (``oracle/liboracle_topk.so``) with g++.

Test infrastructure: only the tests, the smoke check and the benchmark's CPU
baseline load what this builds.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_topk.cpp")
LIB = os.path.join(HERE, "liboracle_topk.so")


def build(verbose: bool = False) -> str:
    # Plain -O3, no -ffast-math and no -march=native: the library built here
    # also runs on other hosts.
    cmd = ["g++", "-O3", "-std=c++17", "-fPIC", "-shared", "-pthread",
           "-fno-fast-math", SRC, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
