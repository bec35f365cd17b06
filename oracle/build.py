"""Build the CPU oracle shared library (test infrastructure only).

Compiles oracle/fairy_oracle.c with gcc into oracle/liboracle.so.  Kept
separate from the HIP library build: the two share no sources or headers.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    src = os.path.join(HERE, "fairy_oracle.c")
    tmp = LIB + ".tmp"
    cmd = [
        "gcc", "-std=gnu11", "-O2", "-fPIC", "-shared", "-fopenmp",
        "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
        "-o", tmp, src, "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
