"""Build the CPU oracle's shared library (test infrastructure; gcc + OpenMP).

Usage: ``python -m oracle.build`` or ``oracle.build.build()``. The library lands next
to this file as ``liboracle.so``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "recurrence.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    """Compile ``recurrence.c`` into ``liboracle.so``; returns the library path."""
    tmp = LIB + ".tmp"
    cmd = ["gcc", "-O3", "-march=x86-64-v3", "-fopenmp", "-fPIC", "-shared",
           "-std=c11", "-Wall", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
