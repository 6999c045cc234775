"""Host-side pieces of bench.py: the one-GPU guard, the name of the timed
kernel instantiation and the hash-gated HBM traffic lookup."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    for args, env in ((["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})):
        out = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                             capture_output=True, text=True, timeout=120,
                             env=dict(os.environ, **env))
        assert out.returncode == 2 and "one GPU" in out.stderr


def test_step_kernel_names_follow_the_launch_policy():
    assert bench.step_kernel_name(8, True) == "step_vec_kernel<8, true, 7, 7, 0, 1>"
    assert bench.step_kernel_name(64, False) == "step_vec_kernel<64, false, 8, 7, 0, 2>"
    assert bench.step_kernel_name(4, True) == "step_vec_kernel<4, true, 3, 7, 0, 1>"
    assert bench.step_kernel_name(32, False) == "step_vec_kernel<32, false, 16, 7, 0, 1>"
    assert bench.step_kernel_name(100, True) == "step_vec_kernel<0, true, 1, 7, 0, 1>"


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    path = os.path.join(ROOT, "profiles", "shard_step_llama8b_traffic.json")
    d = json.load(open(path))
    if d["kernel_hash"] == bench.kernel_hash():
        assert bench.traffic_from_profiles("llama8b", 1.0) == d["hbm_bytes_per_launch"]
    monkeypatch.setattr(bench, "kernel_hash", lambda: "0" * 16)
    assert bench.traffic_from_profiles("llama8b", 1.0) is None
    assert bench.traffic_from_profiles("no_such_workload", 1.0) is None
