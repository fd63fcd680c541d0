"""Builds the oracle's C code into oracle/liboracle.so with the host C compiler.

Test infrastructure: the library it builds is loaded only by oracle/__init__.py.
Plain -O2 (no -ffast-math), so the compiler keeps the fp64 summation order.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["gemm_ref.c", "attn_ref.c"]
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cc = os.environ.get("CC", "gcc")
    tmp = LIB + ".tmp"
    cmd = [cc, "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-fno-fast-math",
           "-ffp-contract=off", "-o", tmp] + [os.path.join(HERE, s) for s in SOURCES] + ["-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
