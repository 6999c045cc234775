"""The C-ABI library on the host: it loads, exports every symbol the header
declares, its layout planner agrees with the oracle's, its per-step scalars
equal the oracle's bit for bit, and bad arguments are rejected before any
GPU work.  No kernel is launched here."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import fsdp_sharded_optimizer_step_amd as z
import oracle
from fsdp_sharded_optimizer_step_amd import binding
from synth import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "zero_shard.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(zero_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = z.load()
    names = header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding.EXPORTS)


def test_package_has_no_oracle_or_fallback_imports():
    pkg = os.path.join(ROOT, "fsdp_sharded_optimizer_step_amd")
    for fn in os.listdir(pkg):
        if fn.endswith(".py"):
            src = open(os.path.join(pkg, fn)).read()
            assert "oracle" not in src, fn
            assert "import synth" not in src, fn


def _layout_matches(numel, cap, n_d):
    pl = oracle.plan(numel, cap, n_d)
    for r in range(n_d):
        L = z.Layout(numel, cap, n_d, r)
        assert (L.psi, L.padded, L.shard, L.n_buckets) == (sum(numel), pl.padded_total,
                                                           pl.shard_len, pl.n_buckets)
        got = np.array(L.buckets(), dtype=np.int64).reshape(-1, 5)
        exp = np.stack([pl.stream_off, pl.len, pl.padded_off, pl.padded_len, pl.shard_off], 1)
        assert np.array_equal(got, exp)
        lo, hi = pl.tensor_ranges(r)
        for t in range(len(numel)):
            so, a, b = L.tensor(t)
            assert so == sum(numel[:t])
            assert (a, b) == (lo[t], hi[t]) or (a == b and lo[t] == hi[t])


@pytest.mark.parametrize("seed", range(30))
def test_layout_agrees_with_oracle_random(seed):
    rng = np.random.default_rng(1000 + seed)
    numel = [int(v) for v in rng.integers(0, 60, int(rng.integers(1, 9)))]
    cap = int(rng.choice([0, 1, 5, 16, 33, 64, 1000]))
    n_d = int(rng.choice([1, 2, 3, 4, 7, 8, 64]))
    _layout_matches(numel, cap, n_d)


@pytest.mark.parametrize("name", ["flat1m", "gpt2s", "accum1p3b"])
def test_layout_agrees_with_oracle_workloads(name):
    w = workloads.get(name)
    _layout_matches(w.numel, w.cap, w.n_d)


@pytest.mark.parametrize("name", ["llama8b", "llama70b", "llama70b_t"])
def test_layout_agrees_with_oracle_large(name):
    w = workloads.get(name)
    pl = oracle.plan(w.numel, w.cap, w.n_d)
    L = z.Layout(w.numel, w.cap, w.n_d, w.rank)
    assert (L.padded, L.shard, L.n_buckets) == (pl.padded_total, pl.shard_len, pl.n_buckets)
    for b in (0, 1, pl.n_buckets // 2, pl.n_buckets - 1):
        assert L.bucket(b) == (pl.stream_off[b], pl.len[b], pl.padded_off[b], pl.padded_len[b],
                               pl.shard_off[b])
    lo, hi = pl.tensor_ranges(w.rank)
    for t in range(len(w.numel)):
        _, a, b = L.tensor(t)
        assert (a, b) == (lo[t], hi[t]) or (a == b and lo[t] == hi[t])


@pytest.mark.parametrize("seed", range(20))
def test_dim0_layout_agrees_with_oracle(seed):
    rng = np.random.default_rng(3000 + seed)
    n_t = int(rng.integers(1, 8))
    rows = [int(v) for v in rng.integers(0, 40, n_t)]
    per_row = [int(v) for v in rng.integers(1, 9, n_t)]
    numel = [r * k for r, k in zip(rows, per_row)]
    n_d = int(rng.choice([1, 2, 3, 4, 8, 64]))
    pl = oracle.plan(numel, 0, n_d, rows=rows)
    for r in range(n_d):
        L = z.Layout(numel, 0, n_d, r, rows=rows)
        assert L.kind == 1
        assert (L.psi, L.padded, L.shard, L.n_buckets) == (sum(numel), pl.padded_total,
                                                           pl.shard_len, pl.n_buckets)
        got = np.array(L.buckets(), dtype=np.int64).reshape(-1, 5)
        exp = np.stack([pl.stream_off, pl.len, pl.padded_off, pl.padded_len, pl.shard_off], 1)
        assert np.array_equal(got, exp)
        lo, hi = pl.tensor_ranges(r)
        for t in range(n_t):
            _, a, b = L.tensor(t)
            assert (a, b) == (lo[t], hi[t]) or (a == b and lo[t] == hi[t])


def test_dim0_layout_errors():
    lib = z.load()
    h = C.c_void_p()
    numel = (C.c_int64 * 2)(8, 9)
    rows = (C.c_int64 * 2)(4, 2)       # 9 is not a multiple of 2
    assert lib.zero_layout_create_dim0(numel, rows, 2, 2, 0, C.byref(h)) == z.binding.ZERO_EINVAL
    rows0 = (C.c_int64 * 2)(4, 0)      # zero rows with elements
    assert lib.zero_layout_create_dim0(numel, rows0, 2, 2, 0, C.byref(h)) == z.binding.ZERO_EINVAL
    ok = (C.c_int64 * 2)(4, 3)
    assert lib.zero_layout_create_dim0(numel, ok, 2, 2, 2, C.byref(h)) == z.binding.ZERO_ERANGE
    assert lib.zero_layout_create_dim0(numel, ok, 2, 0, 0, C.byref(h)) == z.binding.ZERO_EINVAL
    assert z.Layout([8, 9], 0, 2, 0).kind == 0


@pytest.mark.parametrize("t", [1, 2, 10, 101, 1001, 10 ** 6])
@pytest.mark.parametrize("hp", [dict(), dict(lr=3e-4, beta1=0.8, beta2=0.999, eps=1e-6,
                                             weight_decay=0.0), dict(beta1=0.0, beta2=0.0)])
def test_step_scalars_equal_oracle(t, hp):
    got = np.array(z.zero_step_scalars(z.AdamW(**hp), t), np.float32)
    exp = oracle.step_scalars(oracle.AdamW(**hp), t)
    assert np.array_equal(got.view(np.uint32), exp.view(np.uint32))


def test_layout_errors():
    lib = z.load()
    h = C.c_void_p()
    arr = (C.c_int64 * 2)(5, 7)
    assert lib.zero_layout_create(arr, 2, 4, 0, 0, C.byref(h)) == z.binding.ZERO_EINVAL
    assert lib.zero_layout_create(arr, 2, 4, 257, 0, C.byref(h)) == z.binding.ZERO_EINVAL
    assert lib.zero_layout_create(arr, 2, 4, 4, 4, C.byref(h)) == z.binding.ZERO_ERANGE
    assert lib.zero_layout_create(arr, 2, 4, 4, -1, C.byref(h)) == z.binding.ZERO_ERANGE
    assert lib.zero_layout_create(None, 2, 4, 4, 0, C.byref(h)) == z.binding.ZERO_EINVAL
    neg = (C.c_int64 * 2)(5, -1)
    assert lib.zero_layout_create(neg, 2, 4, 4, 0, C.byref(h)) == z.binding.ZERO_EINVAL
    big = (C.c_int64 * 2)(2 ** 61, 2 ** 61)
    assert lib.zero_layout_create(big, 2, 4, 4, 0, C.byref(h)) == z.binding.ZERO_ERANGE
    L = z.Layout([5, 7], 4, 4, 1)
    with pytest.raises(z.ZeroError):
        L.bucket(L.n_buckets)
    with pytest.raises(z.ZeroError):
        L.tensor(2)
    e = z.Layout([], 4, 4, 1)
    assert (e.psi, e.padded, e.shard, e.n_buckets) == (0, 0, 0, 0)


def test_step_argument_errors_before_launch():
    """Invalid calls fail validation on the host; nothing reaches the GPU."""
    lib = z.load()
    L = z.Layout([64], 0, 2, 0)
    hp = binding._AdamW(1e-3, 0.9, 0.95, 1e-8, 0.1)
    fake = [C.c_void_p(0x1000 * (k + 1)) for k in range(8)]
    g = (C.c_void_p * 2)(0x100000, 0x200000)

    def step(layout=L.handle, hp_=hp, t=1, grads=g, gl=0, master=0x300000, m=0x400000,
             v=0x500000, p=0x600000, om=1, gout=None):
        return lib.zero_shard_step(layout, C.byref(hp_) if hp_ is not None else None, t, grads,
                                   gl, master, m, v, p, om, gout, None)

    E = z.binding
    assert step(layout=None) == E.ZERO_EINVAL
    assert step(hp_=None) == E.ZERO_EINVAL
    assert step(t=0) == E.ZERO_EINVAL
    assert step(gl=2) == E.ZERO_EINVAL
    assert step(om=5) == E.ZERO_EINVAL
    assert step(master=None) == E.ZERO_EINVAL
    assert step(grads=(C.c_void_p * 2)(0x100000, None)) == E.ZERO_EINVAL
    assert step(hp_=binding._AdamW(float("nan"), 0.9, 0.95, 1e-8, 0.1)) == E.ZERO_EINVAL
    assert step(hp_=binding._AdamW(1e-3, 1.0, 0.95, 1e-8, 0.1)) == E.ZERO_EINVAL
    assert step(hp_=binding._AdamW(1e-3, 0.9, -0.1, 1e-8, 0.1)) == E.ZERO_EINVAL
    assert step(hp_=binding._AdamW(1e-3, 0.9, 0.95, float("inf"), 0.1)) == E.ZERO_EINVAL
    # overlapping outputs / inputs
    assert step(m=0x300000 + 16) == E.ZERO_EOVERLAP
    assert step(p=0x500000 + 2) == E.ZERO_EOVERLAP
    assert step(grads=(C.c_void_p * 2)(0x100000, 0x400000 + 4)) == E.ZERO_EOVERLAP
    assert step(gout=0x600000 + 8) == E.ZERO_EOVERLAP
    # bad launch shapes
    bad = binding._Options(0, 0, 100, 0)
    rc = lib.zero_shard_step_ex(L.handle, C.byref(hp), 1, g, 0, 0x300000, 0x400000, 0x500000,
                                0x600000, 1, None, C.byref(bad), None)
    assert rc == E.ZERO_EINVAL
    bad_dtype = binding._Options(7, 0, 0, 0)
    rc = lib.zero_shard_step_ex(L.handle, C.byref(hp), 1, g, 0, 0x300000, 0x400000, 0x500000,
                                0x600000, 1, None, C.byref(bad_dtype), None)
    assert rc == E.ZERO_EINVAL
    # S = 32: 64 bytes of bf16 end just before master, 128 bytes of fp32 reach into it
    g2 = (C.c_void_p * 2)(0x300000 - 64, 0x200000)
    f32opt = binding._Options(1, 0, 0, 0)
    rc = lib.zero_shard_step_ex(L.handle, C.byref(hp), 1, g2, 0, 0x300000, 0x400000, 0x500000,
                                0x600000, 1, None, C.byref(f32opt), None)
    assert rc == E.ZERO_EOVERLAP
    # empty shard: nothing to do, succeeds without touching the GPU
    L0 = z.Layout([], 0, 2, 0)
    assert step(layout=L0.handle) == E.ZERO_OK
    del fake


def test_fused_accumulate_step_argument_errors():
    """zero_shard_step_accumulate validates on the host, like the step."""
    lib = z.load()
    E = z.binding
    L = z.Layout([64], 0, 2, 0)                      # S = 32
    hp = binding._AdamW(1e-3, 0.9, 0.95, 1e-8, 0.1)
    acc = (C.c_void_p * 2)(0x100000, 0x110000)
    mic = (C.c_void_p * 2)(0x200000, 0x210000)

    def call(layout=L.handle, a=acc, g=mic, scale=0.25, dt=0, gl=0, master=0x300000, p=0x600000,
             om=1, opt=None):
        return lib.zero_shard_step_accumulate(layout, C.byref(hp), 1, a, g, scale, dt, gl, master,
                                              0x400000, 0x500000, p, om, None, opt, None)

    assert call(a=None) == E.ZERO_EINVAL
    assert call(g=None) == E.ZERO_EINVAL
    assert call(a=(C.c_void_p * 2)(0x100000, None)) == E.ZERO_EINVAL
    assert call(g=(C.c_void_p * 2)(None, 0x210000)) == E.ZERO_EINVAL
    assert call(dt=2) == E.ZERO_EINVAL
    assert call(scale=float("nan")) == E.ZERO_EINVAL
    assert call(gl=3) == E.ZERO_EINVAL
    assert call(opt=C.byref(binding._Options(0, 0, 96, 0))) == E.ZERO_EINVAL
    # 32 fp32 accumulators are 128 bytes: one that ends 64 bytes into master overlaps it
    assert call(a=(C.c_void_p * 2)(0x300000 - 64, 0x110000)) == E.ZERO_EOVERLAP
    assert call(p=0x210000 + 8) == E.ZERO_EOVERLAP
    big = z.Layout([1000], 0, E.ZERO_MAX_ND_FUSED + 1, 0)
    arr = (C.c_void_p * big.n_d)(*[0x1000000 + 0x10000 * k for k in range(big.n_d)])
    assert call(layout=big.handle, a=arr, g=arr) == E.ZERO_ERANGE
    assert call(layout=z.Layout([], 0, 2, 0).handle) == E.ZERO_OK


def test_bucket_range_step_argument_errors():
    """zero_shard_step_buckets checks its bucket range and then validates
    like zero_shard_step_ex; an empty range succeeds without a launch."""
    lib = z.load()
    E = z.binding
    L = z.Layout([40, 24, 100], 32, 2, 1)            # 5 buckets of 32 and one of 4
    hp = binding._AdamW(1e-3, 0.9, 0.95, 1e-8, 0.1)
    g = (C.c_void_p * 2)(0x100000, 0x200000)

    def call(b0=0, b1=None, grads=g, master=0x300000, m=0x400000, p=0x600000, om=1, opt=None):
        b1 = L.n_buckets if b1 is None else b1
        return lib.zero_shard_step_buckets(L.handle, C.byref(hp), 1, b0, b1, grads, 0, master,
                                           m, 0x500000, p, om, None, opt, None)

    nb = L.n_buckets
    assert call(b0=-1) == E.ZERO_ERANGE
    assert call(b1=nb + 1) == E.ZERO_ERANGE
    assert call(b0=2, b1=1) == E.ZERO_ERANGE
    assert call(b0=1, b1=1) == E.ZERO_OK
    assert call(b0=nb, b1=nb) == E.ZERO_OK
    assert call(b0=0, b1=2, master=None) == E.ZERO_EINVAL
    assert call(b0=0, b1=2, grads=(C.c_void_p * 2)(0x100000, None)) == E.ZERO_EINVAL
    assert call(b0=0, b1=2, m=0x300000 + 16) == E.ZERO_EOVERLAP
    assert call(b0=1, b1=2, opt=C.byref(binding._Options(0, 0, 96, 0))) == E.ZERO_EINVAL
    assert call(b0=1, b1=2, opt=C.byref(binding._Options(5, 0, 0, 0))) == E.ZERO_EINVAL
    assert lib.zero_shard_step_buckets(None, C.byref(hp), 1, 0, 1, g, 0, 0x300000, 0x400000,
                                       0x500000, 0x600000, 1, None, None, None) == E.ZERO_EINVAL


def test_accumulate_and_pack_argument_errors():
    lib = z.load()
    E = z.binding
    assert lib.zero_grad_accumulate(0x1000, 0x2000, -1, 1.0, 0, None, None) == E.ZERO_EINVAL
    assert lib.zero_grad_accumulate(0x1000, 0x2000, 8, 1.0, 8, None, None) == E.ZERO_EINVAL
    assert lib.zero_grad_accumulate(0x1000, 0x2000, 8, 1.0, E.ACC_NO_STORE, None, None) == E.ZERO_EINVAL
    assert lib.zero_grad_accumulate(0x1000, 0x2000, 8, 1.0, E.ACC_EMIT_BF16, None, None) == E.ZERO_EINVAL
    assert lib.zero_grad_accumulate(None, 0x2000, 8, 1.0, 0, None, None) == E.ZERO_EINVAL
    assert lib.zero_grad_accumulate(0x1000, 0x1000 + 4, 8, 1.0, 0, None, None) == E.ZERO_EOVERLAP
    assert lib.zero_grad_accumulate(0x1000, 0x2000, 8, 1.0, E.ACC_EMIT_BF16, 0x2000 + 2,
                                    None) == E.ZERO_EOVERLAP
    assert lib.zero_grad_accumulate(0x1000, 0x2000, 0, 1.0, 0, None, None) == E.ZERO_OK
    L = z.Layout([10, 20], 8, 2, 0)
    arr = (C.c_void_p * 2)(0x10000, None)
    assert lib.zero_bucket_pack(L.handle, arr, 0, 5, 0x20000, None) == E.ZERO_ERANGE
    assert lib.zero_bucket_pack(L.handle, arr, 2, 1, 0x20000, None) == E.ZERO_ERANGE
    assert lib.zero_bucket_pack(L.handle, arr, 0, 2, None, None) == E.ZERO_EINVAL
    # tensor 1 has elements in bucket 1 but its pointer is NULL
    assert lib.zero_bucket_pack(L.handle, arr, 0, 2, 0x20000, None) == E.ZERO_EINVAL
    ov = (C.c_void_p * 2)(0x10000, 0x20000 + 6)
    assert lib.zero_bucket_pack(L.handle, ov, 0, 4, 0x20000, None) == E.ZERO_EOVERLAP
    assert lib.zero_bucket_pack(L.handle, arr, 1, 1, 0x20000, None) == E.ZERO_OK


# ------------------------------------------------------------------ placement planner
def _classes(offs, lane, n_lanes):
    return [(o // lane) % n_lanes for o in offs]


def _check_plan(nbytes, traffic, lane, n_lanes, align):
    offs, total = binding.zero_placement_plan(nbytes, traffic, lane, n_lanes, align)
    iv = sorted((o, o + n) for o, n in zip(offs, nbytes))
    assert all(a[1] <= b[0] for a, b in zip(iv, iv[1:])), "buffers overlap"
    assert all(o % align == 0 for o in offs)
    assert total == (max(o + n for o, n in zip(offs, nbytes)) if nbytes else 0)
    for o, n in zip(offs, nbytes):
        if n <= lane:   # a buffer that fits a lane stays inside one lane slot
            assert o // lane == (o + n - 1) // lane or n == 0
    return offs, total


def test_placement_plan_spreads_the_llama8b_step_over_three_lanes():
    """Contributions (2 B/elem each), fp32 state (8 B/elem each) and the bf16
    output (2 B/elem): the three 32 GiB lane classes carry 14 B/elem each."""
    S, P, GiB = 1_003_782_656, 8_030_261_248, 1 << 30
    for out_bytes in (2 * P, 2 * S):
        nbytes = [2 * S] * 8 + [4 * S] * 3 + [out_bytes]
        traffic = [2.0] * 8 + [8.0] * 3 + [2.0]
        offs, total = _check_plan(nbytes, traffic, 32 * GiB, 3, 2 << 20)
        load = [0.0] * 3
        for c, t in zip(_classes(offs, 32 * GiB, 3), traffic):
            load[c] += t
        assert load == [14.0, 14.0, 14.0]
        # the three state arrays land in three different lanes
        assert sorted(_classes(offs[8:11], 32 * GiB, 3)) == [0, 1, 2]
        assert total < 96 * GiB


def test_placement_plan_llama70b_and_edge_cases():
    S, GiB = 1_102_401_664, 1 << 30
    nbytes = [2 * S] * 64 + [4 * S] * 3 + [2 * S]
    traffic = [2.0] * 64 + [8.0] * 3 + [2.0]
    offs, total = _check_plan(nbytes, traffic, 32 * GiB, 3, 2 << 20)
    load = [0.0] * 3
    for c, t in zip(_classes(offs, 32 * GiB, 3), traffic):
        load[c] += t
    assert max(load) - min(load) <= 2.0
    # deterministic
    assert binding.zero_placement_plan(nbytes, traffic, 32 * GiB, 3, 2 << 20) == (offs, total)
    # a buffer larger than a lane goes after the others
    offs, total = _check_plan([100, 5000, 30], [1.0, 1.0, 1.0], 1024, 3, 16)
    assert offs[1] >= max(offs[0] + 100, offs[2] + 30)
    # one lane: packed in list order
    offs, _ = _check_plan([100, 50, 70], [1.0, 9.0, 3.0], 4096, 1, 16)
    assert offs == [0, 112, 176]
    # nothing to place
    assert binding.zero_placement_plan([], [], 1024, 3, 16) == ([], 0)
    # zero-sized buffers are allowed
    _check_plan([0, 64, 0], [1.0, 2.0, 0.0], 1024, 3, 16)


def test_placement_plan_errors():
    lib = z.load()
    E = z.binding
    nb = (C.c_int64 * 2)(10, 20)
    tr = (C.c_double * 2)(1.0, 2.0)
    offs = (C.c_int64 * 2)()
    tot = C.c_int64()

    def call(n=2, nbytes=nb, traffic=tr, lane=1024, lanes=3, align=16, o=offs, t=C.byref(tot)):
        return lib.zero_placement_plan(n, nbytes, traffic, lane, lanes, align, o, t)

    assert call() == E.ZERO_OK
    assert call(n=-1) == E.ZERO_EINVAL
    assert call(nbytes=None) == E.ZERO_EINVAL
    assert call(o=None) == E.ZERO_EINVAL
    assert call(t=None) == E.ZERO_EINVAL
    assert call(lanes=0) == E.ZERO_EINVAL
    assert call(lanes=65) == E.ZERO_EINVAL
    assert call(align=24) == E.ZERO_EINVAL
    assert call(align=8) == E.ZERO_EINVAL
    assert call(lane=1000) == E.ZERO_EINVAL
    assert call(lane=0) == E.ZERO_EINVAL
    assert call(traffic=(C.c_double * 2)(1.0, float("nan"))) == E.ZERO_EINVAL
    assert call(traffic=(C.c_double * 2)(-1.0, 1.0)) == E.ZERO_EINVAL
    assert call(nbytes=(C.c_int64 * 2)(-5, 1)) == E.ZERO_EINVAL
    assert call(nbytes=(C.c_int64 * 2)(1 << 62, 1)) == E.ZERO_ERANGE
    assert call(n=0, nbytes=None, traffic=None, o=None) == E.ZERO_OK and tot.value == 0
