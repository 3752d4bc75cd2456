"""Writes the stored oracle outputs under tests/golden/.

Calls only the oracle and the seeded input generator; nothing here comes
from the GPU path.  Run from the repository root:

    python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import datagen  # noqa: E402
import oracle   # noqa: E402


def main():
    wl = datagen.workload("m1_n256_k256")
    p = datagen.make_workload(wl)
    c, _, _ = oracle.gemm(p.a, p.w, p.scale, p.m, p.n, p.k)
    path = os.path.join(HERE, wl.name + ".c_bits.txt")
    with open(path, "w") as fh:
        fh.write("# BF16 bits of C for workload %s (seed %d), one row of %d;\n"
                 "# written by tests/golden/make_golden.py from the oracle.\n"
                 % (wl.name, wl.seed, wl.n))
        np.savetxt(fh, c.reshape(1, -1).astype(np.int64), fmt="%d")


if __name__ == "__main__":
    main()
