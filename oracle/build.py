"""Build the oracle shared library (test infrastructure only).

Compiles ``glu_oracle.c`` with the host gcc: fp64 arithmetic, OpenMP over
output positions, no fast math and no FMA contraction, so every rounding the
oracle performs is the one its source spells out.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(HERE, "glu_oracle.c")
LIBRARY = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-O2",
    "-std=c11",
    "-fopenmp",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wextra",
    "-Werror",
]


def build(verbose: bool = False) -> str:
    """Compile the oracle library in place and return its path."""
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", *CFLAGS, "-o", tmp, SOURCE, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
