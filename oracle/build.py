"""Build the CPU oracle library (liboracle.so) with gcc.

TEST INFRASTRUCTURE ONLY.  The oracle is compiled by gcc, never by hipcc,
and shares no source with the HIP library.  -ffp-contract=off keeps every
multiply and add separately rounded as written.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "orc.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
