"""Build the CPU oracle library (test infrastructure) with the system C compiler.

Flags: -O2 for speed, -ffp-contract=off so that no multiply-add is fused
except the explicit fmaf() calls, no fast-math, so fp32 division and rounding
follow IEEE 754."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-Wall", "-Wextra", "-o", LIB + ".tmp", os.path.join(HERE, "oracle.c"), "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
