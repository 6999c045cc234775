"""The C ABI from a plain C program: tests/abi_c_smoke.c is compiled with gcc
as C11 against include/zero_shard.h, linked to the built library and run
(host-side entry points only)."""
import os
import subprocess

import fsdp_sharded_optimizer_step_amd as z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_plain_c_client(tmp_path):
    lib_dir = os.path.dirname(z.binding.LIB_PATH)
    assert os.path.exists(z.binding.LIB_PATH), "library not built"
    exe = str(tmp_path / "abi_c_smoke")
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    os.path.join(ROOT, "tests", "abi_c_smoke.c"), "-L", lib_dir, "-lzero_shard",
                    f"-Wl,-rpath,{lib_dir}", "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "ok"
