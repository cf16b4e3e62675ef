"""Build the CPU oracle (test infrastructure) as a shared library with the host compiler.

Plain C++17, fp64, no fast-math and no FMA contraction, so every rounding is the one the
source spells out.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "twilight_oracle.cpp")
OUT = os.path.join(HERE, "liboracle_twilight.so")


def build(verbose: bool = False) -> str:
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-Wall", "-Wextra", "-o", OUT + ".tmp", SRC]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
