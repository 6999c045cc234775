"""Compile the synthetic-input generator (host + gfx950 device code) into
synth/libsynth.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "synth_gen.hip")
OUT = os.path.join(HERE, "libsynth.so")

FLAGS = ["--offload-arch=gfx950", "-std=c++17", "-O3", "-fPIC", "-shared", "-pthread",
         "-ffp-contract=off", "-fno-fast-math",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, SRC, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
