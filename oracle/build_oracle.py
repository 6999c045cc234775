"""Compile the CPU oracle (test infrastructure) into oracle/liboracle.so.

Plain g++, -O2, no fast-math, no FMA contraction, so every binary32 operation
in the oracle is one IEEE-754 operation rounded to nearest-even.
"""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "zero_oracle.cpp")
OUT = os.path.join(HERE, "liboracle.so")

FLAGS = ["-std=c++17", "-O2", "-fPIC", "-shared", "-pthread",
         "-ffp-contract=off", "-fno-fast-math", "-fno-finite-math-only",
         "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    cmd = ["g++", *FLAGS, SRC, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
