"""Builds the oracle's C helper (oracle/libfp8dot.so) with gcc.

TEST INFRASTRUCTURE ONLY: the library is loaded by oracle.lowp to evaluate
its fp8 dot-product model quickly; nothing on the product path uses it.
"""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "fp8_dot.c")
LIB = os.path.join(HERE, "libfp8dot.so")


def build(verbose: bool = True) -> str:
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build()
