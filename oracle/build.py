"""Compile the CPU oracle (plain C, gcc, no HIP) into ``oracle/libmoe_ref.so``.

Test infrastructure: the oracle is built so the tests, the smoke check and the
benchmark's CPU-baseline leg can load it; the HIP library never links it.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "moe_ref.c")
LIB = os.path.join(HERE, "libmoe_ref.so")


def build(verbose: bool = False) -> str:
    """Compile the oracle every time it is called; return the library path."""
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off",
           "-fPIC", "-shared", "-Wall", "-Wextra", "-o", LIB + ".tmp", SRC,
           "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
