"""Build the C-ABI library libzero_shard.so (HIP kernels for gfx950 + host
core) in-tree, next to this file."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libzero_shard.so")
SOURCES = ["layout.cpp", "placement.cpp", "shard_step.hip", "pack_accumulate.hip",
           "gather_reshard.hip"]

# Floating point: no contraction into FMA, correctly rounded binary32 divide
# and square root, subnormals kept (no flush), no fast-math.  Packed fp32
# instructions are disabled for all device code.
FLAGS = ["--offload-arch=gfx950", "-std=c++17", "-O3", "-fPIC", "-shared",
         "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
         "-fno-gpu-flush-denormals-to-zero",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I", os.path.join(ROOT, "include")]


def build(verbose: bool = False, extra=()) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = ["/opt/rocm/bin/hipcc", *FLAGS, *extra, *srcs, "-o", OUT + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(OUT + ".tmp", OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
