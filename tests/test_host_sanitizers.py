"""The library's host code (layout and placement planners) under AddressSanitizer
and UndefinedBehaviorSanitizer: tests/host_sanitize_driver.cpp is built with
g++ together with the two host sources and run on random and edge-case
arguments."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fsdp_sharded_optimizer_step_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = str(tmp_path / "host_sanitize_driver")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
                    os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "placement.cpp"),
                    "-o", exe], check=True)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300,
                         env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert out.returncode == 0, out.stderr[-4000:]
    assert out.stdout.strip() == "ok"
