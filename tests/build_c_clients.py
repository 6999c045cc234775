"""Build the plain C11 clients of the C ABI (tests/abi_c_smoke.c: host-side
entry points; tests/abi_c_step.c: three shard steps on the GPU with hipMalloc'd
memory) into tests/c_bin/, linked to the in-tree libzero_shard.so.  Called by
__graft_entry__.build(); the tests use these executables."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BIN = os.path.join(HERE, "c_bin")
LIB_DIR = os.path.join(ROOT, "fsdp_sharded_optimizer_step_amd")


def exe_path(name: str) -> str:
    return os.path.join(BIN, name)


def build_one(name: str, out: str, with_hip: bool) -> str:
    cmd = ["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           os.path.join(HERE, name + ".c"), "-L", LIB_DIR, "-lzero_shard",
           "-Wl,-rpath,$ORIGIN/../../fsdp_sharded_optimizer_step_amd"]
    if with_hip:
        cmd += ["-L", "/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib"]
    subprocess.run(cmd + ["-o", out + ".tmp"], check=True)
    os.replace(out + ".tmp", out)
    return out


def build() -> None:
    os.makedirs(BIN, exist_ok=True)
    build_one("abi_c_smoke", exe_path("abi_c_smoke"), with_hip=False)
    build_one("abi_c_step", exe_path("abi_c_step"), with_hip=True)


if __name__ == "__main__":
    build()
