"""The C ABI from plain C programs compiled with gcc as C11 against
include/zero_shard.h and linked to the built library (tests/build_c_clients.py,
run by __graft_entry__.build()): tests/abi_c_smoke.c (host-side entry points,
CPU) and tests/abi_c_step.c (three shard steps on the GPU with hipMalloc'd
memory, compared with the CPU oracle)."""
import os
import subprocess

import numpy as np
import pytest

import fsdp_sharded_optimizer_step_amd as z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _client(name):
    """The prebuilt client (built by __graft_entry__.build())."""
    import build_c_clients
    exe = build_c_clients.exe_path(name)
    assert os.path.exists(exe), f"{exe} is not built; run __graft_entry__.build()"
    return exe


def test_plain_c_client():
    assert os.path.exists(z.binding.LIB_PATH), "library not built"
    out = subprocess.run([_client("abi_c_smoke")], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    assert out.stdout.strip() == "ok"


@pytest.mark.gpu
def test_plain_c_client_runs_the_step_on_the_gpu(tmp_path):
    import oracle
    exe = _client("abi_c_step")
    path = str(tmp_path / "out.bin")
    out = subprocess.run([exe, path], capture_output=True, text=True, timeout=120)
    assert out.returncode == 0, out.stderr
    raw = open(path, "rb").read()
    S = int(np.frombuffer(raw[:8], np.int64)[0])
    off = 8

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw[off:off + n * np.dtype(dtype).itemsize], dtype).copy()
        off += n * np.dtype(dtype).itemsize
        return a

    g = take(np.uint16, 4 * S).reshape(4, S)
    st = take(np.float32, 3 * S).reshape(3, S)
    got_st = take(np.float32, 3 * S).reshape(3, S)
    got_p = take(np.uint16, S)
    got_g = take(np.float32, S)
    master, m, v = st[0].copy(), st[1].copy(), st[2].copy()
    hp = oracle.AdamW(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1)
    for t in (1, 2, 3):
        p, ga = oracle.shard_step(list(g), master, m, v, hp, t, want_grad=True)
    for a, b, what in ((got_st[0], master, "master"), (got_st[1], m, "m"), (got_st[2], v, "v"),
                       (got_p, p, "param"), (got_g, ga, "reduced gradient")):
        assert np.array_equal(a.view(np.uint8), np.ascontiguousarray(b).view(np.uint8)), what
