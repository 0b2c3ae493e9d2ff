"""Build the CPU oracle (test infrastructure) into oracle/libmoe_oracle.so with gcc.

The oracle is plain C99 with optional OpenMP over output rows; it is compiled
on its own, from its own sources, and shares nothing with the HIP library.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libmoe_oracle.so")
SRC = [os.path.join(HERE, "moe_oracle.c")]


def build(verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", LIB + ".tmp"] + SRC + ["-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


def ensure_built() -> str:
    if not os.path.exists(LIB):
        build()
    return LIB


if __name__ == "__main__":
    build(verbose="-v" in sys.argv)
    print(LIB)
