"""Build the CPU oracle (test infrastructure) into oracle/liboracle.so.

The oracle is plain C compiled by gcc with contraction and fast-math off, so
its floating-point steps are exactly the ones written in mxref.c.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
           "-fno-math-errno", "-Wall", "-Wextra", "-fPIC", "-shared",
           "-o", LIB + ".tmp", os.path.join(HERE, "mxref.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
