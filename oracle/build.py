"""Compile the fp64 CPU oracle (``ssd_oracle.c``) into ``libssd_oracle.so``.

Test infrastructure only: the GPU library never links or loads the result.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "ssd_oracle.c")
LIB = os.path.join(HERE, "libssd_oracle.so")

# Plain IEEE fp64: no fast-math, no FMA contraction, baseline x86-64 so the
# library also runs on a host CPU other than the one that built it.
CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-Wall", "-Wextra"]


def build_oracle(verbose: bool = False) -> str:
    """Compile the oracle with gcc; returns the library path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build_oracle(verbose=True))
