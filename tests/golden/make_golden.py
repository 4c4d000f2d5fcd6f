"""Writes tests/golden/oracle_small.txt from the fp64 oracle alone.

The pages print no worked example for the token mixer, so this fixture is a
regression snapshot of the oracle (already pinned by brute force and closed
forms in tests/test_oracle.py), not a value from the pages.  Input: the seeded
generator of workloads.py, B=1, N=24 (grid 2x3x4), H=2, D=32, seed 123,
RoPE on with theta = 1e4, eps = 1e-6.

Run from the repository root:  python tests/golden/make_golden.py
"""
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from workloads import random_inputs  # noqa: E402

PATH = os.path.join(HERE, "oracle_small.txt")
SHAPE = (1, 24, 2, 32)


def compute() -> np.ndarray:
    q, k, v, g = random_inputs(*SHAPE, seed=123)
    return oracle.forward(q, k, v, g, oracle.Grid(2, 3, 4))


def read() -> np.ndarray:
    return np.loadtxt(PATH, dtype=np.float64).reshape(SHAPE)


if __name__ == "__main__":
    out = compute()
    np.savetxt(PATH, out.reshape(-1, SHAPE[-1]), fmt="%.17e",
               header="oracle output o[b, n, h, :], rows in (b, n, h) order; see make_golden.py")
    print("wrote", PATH)
