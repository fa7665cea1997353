"""Build the C oracle library (test infrastructure only).

    python -m oracle.build        # writes oracle/libgdn_oracle.so

Portable x86-64-v3 code so that a library built in one container runs on any
AVX2 host; no fast-math, so the fp64 arithmetic follows the source.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gdn_recurrence.c")
LIB = os.path.join(HERE, "libgdn_oracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
