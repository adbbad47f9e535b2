"""Write tests/golden/c1_codes.txt from the oracle (only oracle/ and synthetic/ are used).

The pages print no worked example of the method, so the only stored values are
oracle outputs for the tiny 32x32 workload, cross-checked at write time against
brute-force Babai nearest plane on the 1024-dimensional Kronecker lattice.
Run:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from synthetic import make  # noqa: E402


def main():
    wl = make("C1")
    out = oracle.quantize(wl.W, wl.A, wl.B, wl.scales, wl.bits)
    zb = oracle.babai_nearest_plane(wl.W, wl.A, wl.B, wl.scales, wl.bits)
    assert np.array_equal(out["Z"], zb), "oracle and brute-force Babai disagree"
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c1_codes.txt")
    with open(path, "w") as f:
        f.write("# GPTQ-2D codes for workload C1 (32x32, 4-bit, seed 101), row-major.\n")
        f.write("# Written by tests/golden/make_golden.py from the oracle; equal to\n")
        f.write("# brute-force Babai nearest plane on the 1024-dim Kronecker lattice.\n")
        for row in out["Z"]:
            f.write(" ".join(str(int(v)) for v in row) + "\n")
    print("wrote", path)


if __name__ == "__main__":
    main()
