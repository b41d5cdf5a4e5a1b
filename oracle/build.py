"""Compile the CPU oracle (``oracle.c``) into ``liboracle.so`` with gcc.

Test infrastructure only: the oracle is the checker of the GPU library and is
never linked into it.  Flags: ``-O2 -fno-fast-math -ffp-contract=off`` so that
every float operation the oracle writes is one IEEE single-precision
operation, rounded to nearest even; OpenMP only splits rows over threads.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

CFLAGS = [
    "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
    "-fexcess-precision=standard", "-msse2", "-mfpmath=sse", "-fopenmp", "-Wall", "-Wextra",
]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", *CFLAGS, SRC, "-o", LIB + ".tmp", "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
