"""Write ``oracle_tiny.txt``: the oracle's outputs on one tiny seeded input.

This script calls only ``oracle/`` and the seeded generator.  The file it writes
is a regression fixture for the oracle (it catches an unintended change to the
oracle's arithmetic); the pages print no worked numeric example, so no stored
value here comes from them.
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from ssd_chunked_scan_amd import workloads as wl  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.txt")


def tiny_inputs():
    return wl.make_inputs(1, 20, 2, 2, 3, 1, 8, "fp32", seed=2024, init_std=0.5)


def main():
    inp = tiny_inputs()
    out = oracle.forward(inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.initial_states)
    with open(OUT, "w") as f:
        f.write("# oracle outputs for make_inputs(1, 20, 2, 2, 3, 1, 8, 'fp32', seed=2024, init_std=0.5)\n")
        f.write("# written by tests/golden/make_golden.py (calls only oracle/)\n")
        f.write("# y [1,20,2,2] flattened\n")
        f.write(" ".join(f"{v:.17g}" for v in out.y.reshape(-1)) + "\n")
        f.write("# final_states [1,2,2,3] flattened\n")
        f.write(" ".join(f"{v:.17g}" for v in out.final_states.reshape(-1)) + "\n")
    print(OUT)


if __name__ == "__main__":
    main()
