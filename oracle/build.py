"""Build the CPU fp64 attention reference (test infrastructure only).

Compiles oracle.c with gcc into liboracle.so next to this file. Plain -O2
for the baseline x86-64 ISA (no -march=native, no -ffast-math): the library
built here also runs on other hosts, and IEEE semantics are kept.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "liboracle.so")


def build(verbose: bool = False) -> str:
    cmd = [
        "gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
        "-Wall", "-Wextra", "-Werror",
        os.path.join(HERE, "oracle.c"), "-o", LIB + ".tmp", "-lm",
    ]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
