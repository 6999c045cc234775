"""Compile the same-mix streaming ceiling kernel into measure/libmeasure.so."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "stream_ceiling.hip")
OUT = os.path.join(HERE, "libmeasure.so")
FLAGS = ["--offload-arch=gfx950", "-std=c++17", "-O3", "-fPIC", "-shared",
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
