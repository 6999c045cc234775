"""Pins for the CPU oracle: each test checks it against something other than
itself -- the pages' worked example, closed forms, a library routine,
an exact evaluation within a derived rounding bound, or brute force on tiny
inputs.  CPU only.

Sources: "Infra: Data Parallel" (pufanyi.com) sections "Naive Data
Parallelism", "Zero Redundancy Optimizer (ZeRO)" and "Fully Sharded Data
Parallel (FSDP)" / "FSDP1"; "FSDP" knowledge card (kongchang.com), Core Facts
(float accumulation order must be fixed for determinism).
"""
import json
import os
from concurrent.futures import ThreadPoolExecutor
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
U = 2.0 ** -24  # unit roundoff of binary32


def bf16_of(x):
    """float values -> bf16 bits by torch's own float32->bfloat16 conversion."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# ------------------------------------------------------------------ cast
def test_bf16_round_exhaustive_vs_torch():
    """All 2^32 binary32 patterns: the oracle's round-to-nearest-even equals
    torch's float32->bfloat16 conversion (a library routine); NaNs stay NaN
    with their sign."""
    chunk = 1 << 26

    def one(c):
        lo = c * chunk
        got = oracle.round_bf16_patterns(lo, lo + chunk)
        pats = np.arange(lo, lo + chunk, dtype=np.uint64).astype(np.uint32)
        x = pats.view(np.float32)
        ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        nan = np.isnan(x)
        bad = (got != ref) & ~nan
        if bad.any():
            k = np.flatnonzero(bad)[0]
            return f"pattern {int(pats[k]):#010x}: oracle {int(got[k]):#06x} torch {int(ref[k]):#06x}"
        g = got[nan]
        if not (((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)).all():
            return "NaN did not stay NaN"
        if not (((g >> 15) & 1) == ((pats[nan] >> 31) & 1)).all():
            return "NaN sign lost"
        return None

    with ThreadPoolExecutor(8) as ex:
        errs = [e for e in ex.map(one, range((1 << 32) // chunk)) if e]
    assert not errs, errs[:3]


def test_bf16_round_ties_and_overflow():
    # exact ties: 1 + 2^-8 sits halfway between bf16 1.0 and 1+2^-7 -> even (1.0)
    big = np.array([0x7F7F8000, 0x7F7F7FFF], np.uint32).view(np.float32)  # midpoint, just below
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), big[0], big[1]], dtype=np.float32)
    got = oracle.round_bf16(x)
    assert got[0] == 0x3F80 and got[1] == 0x3F82 and got[2] == 0xBF80
    assert got[3] == 0x7F80          # the midpoint to 2^128 ties to 'even': infinity
    assert got[4] == 0x7F7F          # below it: the largest finite bf16


# ------------------------------------------------------------------ layout
def _brute_layout(numel, cap, n_d):
    """Element-by-element planner written independently of the oracle: label
    every stream element, cut, pad, and deal out slices."""
    stream = [(t, e) for t, n in enumerate(numel) for e in range(n)]
    total = len(stream)
    c = total if cap <= 0 else cap
    buckets = [stream[i:i + c] for i in range(0, total, c)] if total else []
    padded = []
    for b in buckets:
        pad = (-len(b)) % n_d
        padded.append(list(b) + [None] * pad)
    flat = [x for b in padded for x in b]
    shards = []
    for r in range(n_d):
        sh = []
        for b in padded:
            s = len(b) // n_d
            sh += b[r * s:(r + 1) * s]
        shards.append(sh)
    return buckets, padded, flat, shards


@pytest.mark.parametrize("seed", range(40))
def test_layout_brute_force(seed):
    rng = np.random.default_rng(seed)
    n_t = int(rng.integers(1, 7))
    numel = [int(v) for v in rng.integers(0, 14, n_t)]
    cap = int(rng.choice([0, 1, 3, 5, 7, 8, 16, 100]))
    n_d = int(rng.choice([1, 2, 3, 4, 5, 8]))
    buckets, padded, flat, shards = _brute_layout(numel, cap, n_d)
    pl = oracle.plan(numel, cap, n_d)
    assert pl.n_buckets == len(buckets)
    assert pl.padded_total == len(flat) == n_d * pl.shard_len
    assert [len(b) for b in buckets] == list(pl.len)
    assert all(0 <= p - l < n_d for p, l in zip(pl.padded_len, pl.len))
    assert sum(pl.len) == sum(numel)
    # values: label element (t, e) as 1 + 16*t + e (fits bf16 bit patterns)
    tensors = [np.array([1 + 16 * t + e for e in range(n)], np.uint16) for t, n in enumerate(numel)]
    label = {(t, e): 1 + 16 * t + e for t, n in enumerate(numel) for e in range(n)}
    packed = oracle.pack(tensors, pl)
    assert list(packed) == [0 if x is None else label[x] for x in flat]
    for r in range(n_d):
        sl = oracle.slice_shard(packed, pl, r)
        assert list(sl) == [0 if x is None else label[x] for x in shards[r]]
        lo, hi = pl.tensor_ranges(r)
        for t in range(n_t):
            pos = [i for i, x in enumerate(shards[r]) if x is not None and x[0] == t]
            if pos:
                assert (lo[t], hi[t]) == (pos[0], pos[-1] + 1)
                # between them only pads: no element of another tensor
                assert all(shards[r][i] is None or shards[r][i][0] == t
                           for i in range(lo[t], hi[t]))
            else:
                assert lo[t] == hi[t]
        if pl.shard_len:
            idx = np.arange(pl.shard_len)
            fpos, spos = pl.map(r, idx)
            for i in range(pl.shard_len):
                x = shards[r][i]
                assert flat[fpos[i]] == x
                if x is None:
                    assert spos[i] == -1
                else:
                    assert stream_index(numel, x) == spos[i]


@pytest.mark.parametrize("seed", range(25))
def test_gather_locate_reshard_brute_force(seed):
    """Gather is the inverse of slicing; locate and reshard agree with the
    element-by-element planner (labels = stream position + 1, pads = 0)."""
    rng = np.random.default_rng(500 + seed)
    numel = [int(v) for v in rng.integers(0, 14, int(rng.integers(1, 6)))]
    if sum(numel) == 0:
        numel[0] = 3
    cap = int(rng.choice([0, 1, 3, 5, 7, 8, 16]))
    n_d = int(rng.choice([1, 2, 3, 4, 5, 8]))
    _, _, flat, shards = _brute_layout(numel, cap, n_d)
    pl = oracle.plan(numel, cap, n_d)
    lab = lambda x: 0 if x is None else stream_index(numel, x) + 1  # noqa: E731
    sh = [np.array([lab(x) for x in shards[r]], np.uint16) for r in range(n_d)]
    assert list(oracle.gather(sh, pl)) == [lab(x) for x in flat]
    xs = np.arange(sum(numel))
    r, i = oracle.locate(pl, xs)
    for x in xs:
        assert lab(shards[r[x]][i[x]]) == x + 1
    # reshard to another random layout of the same tensors
    cap2 = int(rng.choice([0, 2, 4, 6, 9]))
    n_d2 = int(rng.choice([1, 2, 3, 6]))
    _, _, _, shards2 = _brute_layout(numel, cap2, n_d2)
    pl2 = oracle.plan(numel, cap2, n_d2)
    shf = [a.astype(np.float32) for a in sh]
    for r2 in range(n_d2):
        got = oracle.reshard(shf, pl, pl2, r2)
        assert list(got) == [float(lab(x)) for x in shards2[r2]]
    back = [oracle.reshard([oracle.reshard(shf, pl, pl2, q) for q in range(n_d2)], pl2, pl, r)
            for r in range(n_d)]
    for a, b in zip(back, shf):
        assert np.array_equal(a, b)
    same = [oracle.reshard(sh, pl, pl, r) for r in range(n_d)]
    for a, b in zip(same, sh):
        assert np.array_equal(a, b)


def stream_index(numel, x):
    t, e = x
    return sum(numel[:t]) + e


def test_layout_fsdp1_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "fsdp1_flatparam.json")))
    numel = [int(np.prod(s)) for s in g["shapes"]]
    pl = oracle.plan(numel, 0, g["n_d"])
    assert pl.padded_total == g["padded_total"] and pl.shard_len == g["shard_len"]
    names = g["names"]
    tensors = [np.arange(1, n + 1, dtype=np.uint16) + 100 * k for k, n in enumerate(numel)]
    packed = oracle.pack(tensors, pl)
    for r, pieces in g["ranks"].items():
        r = int(r)
        expect = np.concatenate([tensors[names.index(nm)][a:b] for nm, a, b in pieces])
        assert np.array_equal(oracle.slice_shard(packed, pl, r), expect)
        lo, hi = pl.tensor_ranges(r)
        pos = 0
        for nm, a, b in pieces:
            t = names.index(nm)
            assert (lo[t], hi[t]) == (pos, pos + b - a)
            pos += b - a
        held = {names.index(nm) for nm, _, _ in pieces}
        for t in range(len(names)):
            if t not in held:
                assert lo[t] == hi[t]  # the rank holds none of this tensor: empty view


def _brute_dim0(shapes, n_d):
    """FSDP2 per-parameter layout, element by element: tensor t of shape
    (rows, ...) gives rank r rows [r*c, (r+1)*c), c = ceil(rows/n_d), with
    missing rows as padding; a rank's shard is its pieces in tensor order;
    the gathered buffer holds each tensor padded to n_d*c rows."""
    flat, shards = [], [[] for _ in range(n_d)]
    for t, shp in enumerate(shapes):
        rows = shp[0]
        per_row = int(np.prod(shp[1:])) if len(shp) > 1 else 1
        c = -(-rows // n_d)
        for r in range(n_d):
            for row in range(r * c, (r + 1) * c):
                for k in range(per_row):
                    x = (t, row * per_row + k) if row < rows else None
                    shards[r].append(x)
                    flat.append(x)
    return flat, shards


def test_fsdp2_worked_examples():
    """The FSDP2 figure and text: three (4, 2) weights over 2 ranks give each
    rank the first / last two rows of every weight, local shape (2, 2), 12
    elements per rank; an (8, 4) weight over 4 ranks has local shape (2, 4)."""
    g = json.load(open(os.path.join(GOLDEN, "fsdp2_shard0.json")))
    for case in g["cases"]:
        shapes = [tuple(x) for x in case["shapes"]]
        n_d = case["n_d"]
        numel = [int(np.prod(x)) for x in shapes]
        pl = oracle.plan(numel, 0, n_d, rows=[x[0] for x in shapes])
        assert pl.shard_len == case["elems_per_rank"]
        for t, (shp, loc) in enumerate(zip(shapes, case["local_shapes"])):
            assert pl.padded_len[t] // n_d == int(np.prod(loc))
        tensors = [np.arange(1, n + 1, dtype=np.uint16) + 100 * t for t, n in enumerate(numel)]
        flat = oracle.pack(tensors, pl)
        for r in range(n_d):
            shard = oracle.slice_shard(flat, pl, r)
            rr = case.get("rank_rows", {}).get(str(r))
            if rr:
                expect = np.concatenate([tensors[t].reshape(shapes[t])[a:b].ravel()
                                         for t, (a, b) in enumerate(rr)])
                assert np.array_equal(shard, expect)
            lo, hi = pl.tensor_ranges(r)
            for t, shp in enumerate(shapes):
                assert hi[t] - lo[t] == int(np.prod(case["local_shapes"][t]))


@pytest.mark.parametrize("seed", range(25))
def test_fsdp2_layout_brute_force(seed):
    rng = np.random.default_rng(700 + seed)
    n_t = int(rng.integers(1, 5))
    shapes = [tuple(int(v) for v in rng.integers(1, 7, int(rng.integers(1, 3)))) for _ in range(n_t)]
    if rng.random() < 0.3:
        shapes.append((0, 3))
    n_d = int(rng.choice([1, 2, 3, 4, 5, 8]))
    numel = [int(np.prod(x)) for x in shapes]
    flat, shards = _brute_dim0(shapes, n_d)
    pl = oracle.plan(numel, 0, n_d, rows=[x[0] for x in shapes])
    assert pl.padded_total == len(flat) == n_d * pl.shard_len
    lab = {(t, e): 1 + 16 * t + e for t, n in enumerate(numel) for e in range(n)}
    tensors = [np.array([lab[(t, e)] for e in range(n)], np.uint16) for t, n in enumerate(numel)]
    packed = oracle.pack(tensors, pl)
    assert list(packed) == [0 if x is None else lab[x] for x in flat]
    for r in range(n_d):
        assert list(oracle.slice_shard(packed, pl, r)) == [0 if x is None else lab[x]
                                                          for x in shards[r]]
        if pl.shard_len:
            fpos, spos = pl.map(r, np.arange(pl.shard_len))
            for i, x in enumerate(shards[r]):
                assert flat[fpos[i]] == x
                assert spos[i] == (-1 if x is None else stream_index(numel, x))
    sh = [oracle.slice_shard(packed, pl, r) for r in range(n_d)]
    assert np.array_equal(oracle.gather(sh, pl), packed)
    # re-cut between the dim-0 layout and a bucketed one, both ways
    pb = oracle.plan(numel, 5, 3)
    shf = [a.astype(np.float32) for a in sh]
    there = [oracle.reshard(shf, pl, pb, q) for q in range(3)]
    back = [oracle.reshard(there, pb, pl, r) for r in range(n_d)]
    for a, b in zip(back, shf):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("seed", range(20))
def test_fsdp2_slices_agree_with_torch_chunk(seed):
    """The per-parameter reading (rank r owns rows [r*c, (r+1)*c) with
    c = ceil(rows/N_d), missing rows are padding) is PyTorch's chunk-then-pad
    convention: the real part of rank r's slice of every tensor is
    torch.chunk(t, N_d, dim=0)[r] (or nothing when chunk returns fewer
    pieces), the rest of the slice is zero padding."""
    import torch
    rng = np.random.default_rng(900 + seed)
    shapes = [tuple(int(v) for v in rng.integers(1, 11, int(rng.integers(1, 3))))
              for _ in range(int(rng.integers(1, 6)))]
    n_d = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 16]))
    numel = [int(np.prod(x)) for x in shapes]
    pl = oracle.plan(numel, 0, n_d, rows=[x[0] for x in shapes])
    offs = np.concatenate([[0], np.cumsum(numel)])
    values = [np.arange(1 + offs[t], 1 + offs[t] + n, dtype=np.uint16)
              for t, n in enumerate(numel)]
    packed = oracle.pack(values, pl)
    for r in range(n_d):
        shard = oracle.slice_shard(packed, pl, r)
        for t, shp in enumerate(shapes):
            sl = int(pl.padded_len[t]) // n_d
            got = shard[int(pl.shard_off[t]):int(pl.shard_off[t]) + sl]
            chunks = torch.chunk(torch.from_numpy(values[t].astype(np.int64)).reshape(shp), n_d,
                                 dim=0)
            real = chunks[r].reshape(-1).numpy() if r < len(chunks) else np.zeros(0, np.int64)
            assert np.array_equal(got[:real.size].astype(np.int64), real)
            assert not got[real.size:].any()


@pytest.mark.parametrize("name", workloads.NAMES)
def test_layout_workload_sizes_closed_form(name):
    """Fixed-cut buckets: nb = ceil(psi/C), S = (nb-1)*ceil(C/n_d) + ceil(last/n_d)."""
    w = workloads.get(name)
    pl = oracle.plan(w.numel, w.cap, w.n_d)
    psi = w.psi
    c = psi if w.cap <= 0 else w.cap
    nb = -(-psi // c)
    last = psi - (nb - 1) * c
    S = (nb - 1) * (-(-c // w.n_d)) + (-(-last // w.n_d))
    assert (pl.n_buckets, pl.shard_len, pl.padded_total) == (nb, S, w.n_d * S)


def test_workload_parameter_counts():
    # GPT-2 small with wpe and ln_f; Llama-3-8B; Llama-70B (sizes as stated for the workloads)
    assert workloads.get("gpt2s").psi == 124_439_808 and len(workloads.get("gpt2s").numel) == 148
    assert workloads.get("llama8b").psi == 8_030_261_248 and len(workloads.get("llama8b").numel) == 291
    assert workloads.get("llama70b").psi == 70_553_706_496
    assert len(workloads.get("llama70b").numel) == 723


def test_layout_padded_tail_workload():
    """The 12.5M-element cut of the 70B list pads 32 elements per full bucket,
    all of them in the last rank's slice."""
    w = workloads.get("llama70b_t")
    pl = oracle.plan(w.numel, w.cap, w.n_d)
    pads = pl.padded_len - pl.len
    assert (pads[:-1] == 32).all()
    s_full = pl.padded_len[0] // w.n_d
    assert s_full > 32  # so all pads of a full bucket fall in rank 63's slice
    idx = np.concatenate([pl.shard_off[:3, None] + np.arange(s_full)[None, :]]).ravel()
    _, spos = pl.map(63, idx)
    assert ((spos == -1).reshape(3, s_full).sum(axis=1) == 32).all()
    _, spos0 = pl.map(0, idx)
    assert (spos0 >= 0).all()


# ------------------------------------------------------------------ reduce
HP = oracle.AdamW()


def _step(grads, n, t=1, hp=HP, master=None, m=None, v=None):
    master = np.zeros(n, np.float32) if master is None else master
    m = np.zeros(n, np.float32) if m is None else m
    v = np.zeros(n, np.float32) if v is None else v
    p, g = oracle.shard_step(grads, master, m, v, hp, t, want_grad=True)
    return master, m, v, p, g


def test_reduce_rank_order_pin():
    """[1, 2^-24, -1] in rank order gives exactly 0; the reordered sum would be
    2^-24.  (The pages require a fixed accumulation order for determinism.)"""
    vals = np.array([1.0, 2.0 ** -24, -1.0], np.float32)
    grads = [bf16_of(vals[q:q + 1]) for q in range(3)]
    *_, g = _step(grads, 1)
    assert g[0] == 0.0
    swapped = [grads[0], grads[2], grads[1]]
    *_, g2 = _step(swapped, 1)
    assert g2[0] == np.float32(2.0 ** -24 / 3)


def test_reduce_negative_zero_start():
    neg = bf16_of(np.array([-0.0], np.float32))
    for n_d in (1, 2, 8):
        *_, g = _step([neg] * n_d, 1)
        assert np.signbit(g[0]) and g[0] == 0.0


def test_reduce_exact_small_integers():
    """Sums of small integers are exact in fp32: compare with exact rationals."""
    rng = np.random.default_rng(1)
    for n_d in (1, 2, 3, 4, 5, 8, 64):
        vals = rng.integers(-200, 200, size=(n_d, 257)).astype(np.float32)
        grads = [bf16_of(vals[q]) for q in range(n_d)]
        *_, g = _step(grads, 257)
        for k in range(257):
            exact = Fraction(int(vals[:, k].sum()), n_d)
            assert g[k] == np.float32(float(exact))  # float(Fraction) is correctly rounded


def test_reduce_post_divide_equals_pre_divide_pow2():
    rng = np.random.default_rng(2)
    for n_d in (2, 4, 8, 64):
        vals = (rng.standard_normal((n_d, 4096)) * 1e-3).astype(np.float32)
        grads = [bf16_of(vals[q]) for q in range(n_d)]
        *_, g = _step(grads, 4096)
        w = [oracle.widen_bf16(x) for x in grads]
        pre = w[0] / np.float32(n_d)
        for q in range(1, n_d):
            pre = pre + w[q] / np.float32(n_d)
        assert np.array_equal(g.view(np.uint32), pre.view(np.uint32))


def test_f32_contributions_equal_bf16_path_on_bf16_values():
    """fp32 contributions that hold bf16 values give exactly the bf16 path's
    update (the reduction sees the same binary32 numbers)."""
    rng = np.random.default_rng(21)
    n = 5000
    for n_d in (1, 3, 8, 64):
        grads = [bf16_of((rng.standard_normal(n) * 1e-3).astype(np.float32)) for _ in range(n_d)]
        th = (rng.standard_normal(n) * 0.02).astype(np.float32)
        m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32)
        v0 = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32)
        a = [th.copy(), m0.copy(), v0.copy()]
        b = [th.copy(), m0.copy(), v0.copy()]
        pa, ga = oracle.shard_step(grads, *a, HP, 7, want_grad=True)
        pb, gb = oracle.shard_step_f32([oracle.widen_bf16(g) for g in grads], *b, HP, 7,
                                       want_grad=True)
        assert np.array_equal(pa, pb) and np.array_equal(ga.view(np.uint32), gb.view(np.uint32))
        for x, y in zip(a, b):
            assert np.array_equal(x.view(np.uint32), y.view(np.uint32))


def test_f32_reduce_order_and_exact_sums():
    master, m, v = (np.zeros(1, np.float32) for _ in range(3))
    vals = [np.array([1.0], np.float32), np.array([2.0 ** -24], np.float32),
            np.array([-1.0], np.float32)]
    _, g = oracle.shard_step_f32(vals, master, m, v, HP, 1, want_grad=True)
    assert g[0] == 0.0
    rng = np.random.default_rng(22)
    for n_d in (2, 5, 8):
        ints = rng.integers(-10 ** 6, 10 ** 6, size=(n_d, 300))
        G = [ints[q].astype(np.float32) for q in range(n_d)]
        z3 = [np.zeros(300, np.float32) for _ in range(3)]
        _, g = oracle.shard_step_f32(G, *z3, HP, 1, want_grad=True)
        for k in range(300):
            assert g[k] == np.float32(float(Fraction(int(ints[:, k].sum()), n_d)))


# ------------------------------------------------------------------ accumulate
def test_accumulate_four_quarter_micro_batches_equal_full_batch_mean():
    """Four equal micro-batches, each scaled by 1/4 and summed locally, equal
    the mean over the full batch (the sum of the four divided by 4), bitwise."""
    rng = np.random.default_rng(3)
    n = 1 << 16
    micro = [bf16_of(rng.standard_normal(n).astype(np.float32) * 2e-3) for _ in range(4)]
    acc = np.full(n, np.nan, np.float32)  # overwrite must ignore stale contents
    for k in range(4):
        emitted = oracle.accumulate(acc, micro[k], 0.25, overwrite=(k == 0), emit=(k == 3))
    w = [oracle.widen_bf16(x) for x in micro]
    mean = (((w[0] + w[1]) + w[2]) + w[3]) / np.float32(4)
    assert np.array_equal(acc.view(np.uint32), mean.view(np.uint32))
    assert np.array_equal(emitted, bf16_of(mean))
    # a step on the accumulated contribution equals a step on the precomputed mean
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    a = _step([emitted] * 2, n, 5, master=th.copy())
    b = _step([bf16_of(mean)] * 2, n, 5, master=th.copy())
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_accumulate_skip_store_and_emit():
    rng = np.random.default_rng(4)
    n = 999
    g = bf16_of(rng.standard_normal(n).astype(np.float32))
    acc = rng.standard_normal(n).astype(np.float32)
    before = acc.copy()
    out = oracle.accumulate(acc, g, 0.5, overwrite=False, store_acc=False, emit=True)
    assert np.array_equal(acc, before)
    assert np.array_equal(out, bf16_of(before + np.float32(0.5) * oracle.widen_bf16(g)))


# ------------------------------------------------------------------ AdamW
def test_adamw_step1_closed_form():
    """m = v = 0, t = 1: bias correction makes the update
    (1 - lr*wd)*theta - lr*g/(|g| + eps); gate by a rounding bound."""
    rng = np.random.default_rng(5)
    n = 1 << 16
    for n_d in (4, 8, 64):
        vals = (rng.standard_normal((n_d, n)) * 1e-3).astype(np.float32)
        grads = [bf16_of(vals[q]) for q in range(n_d)]
        th = (rng.standard_normal(n) * 0.02).astype(np.float32)
        master, m, v, p, g = _step(grads, n, 1, master=th.copy())
        g64 = g.astype(np.float64)
        awd = (1 - HP.lr * HP.weight_decay) * th.astype(np.float64)
        u = HP.lr * g64 / (np.abs(g64) + HP.eps)
        cf = awd - u
        err = np.abs(master.astype(np.float64) - cf)
        bound = 8 * U * (np.abs(awd) + np.abs(u))
        assert (err <= bound).all(), float((err / bound).max())


def test_adamw_zero_gradient_special_case():
    rng = np.random.default_rng(6)
    n = 4096
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    z = np.zeros(n, np.uint16)
    master, m, v, p, g = _step([z, z], n, 1, master=th.copy())
    awd = np.float32(1 - HP.lr * HP.weight_decay)
    assert np.array_equal(master, awd * th)
    assert not m.any() and not v.any()
    assert np.array_equal(p, bf16_of(awd * th))


def _torch_adamw_f64_one_step(th, m, v, g, t, hp):
    """torch.optim.AdamW (single-tensor loop) in float64 from the given state."""
    p = torch.nn.Parameter(torch.from_numpy(th.astype(np.float64)))
    opt = torch.optim.AdamW([p], lr=hp.lr, betas=(hp.beta1, hp.beta2), eps=hp.eps,
                            weight_decay=hp.weight_decay, foreach=False)
    p.grad = torch.from_numpy(g.astype(np.float64))
    opt.step()  # creates state at step 1
    if t > 1:
        with torch.no_grad():
            p.copy_(torch.from_numpy(th.astype(np.float64)))
        st = opt.state[p]
        st["step"] = torch.tensor(float(t - 1), dtype=torch.float64)
        st["exp_avg"].copy_(torch.from_numpy(m.astype(np.float64)))
        st["exp_avg_sq"].copy_(torch.from_numpy(v.astype(np.float64)))
        opt.step()
    st = opt.state[p]
    return p.detach().numpy(), st["exp_avg"].numpy(), st["exp_avg_sq"].numpy()


@pytest.mark.parametrize("t", [1, 2, 10, 101, 1001])
def test_adamw_vs_torch_float64_within_rounding_bound(t):
    """One step from the same state: the fp32 oracle is within a derived
    binary32 rounding bound of torch.optim.AdamW evaluated in float64."""
    rng = np.random.default_rng(100 + t)
    n = 1 << 15
    n_d = 8
    vals = (rng.standard_normal((n_d, n)) * 1e-3).astype(np.float32)
    grads = [bf16_of(vals[q]) for q in range(n_d)]
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(n) * 1e-4).astype(np.float32) if t > 1 else np.zeros(n, np.float32)
    v0 = np.abs(rng.standard_normal(n) * 1e-6).astype(np.float32) if t > 1 else np.zeros(n, np.float32)
    master, m, v, p, g = _step(grads, n, t, master=th.copy(), m=m0.copy(), v=v0.copy())
    rt, rm, rv = _torch_adamw_f64_one_step(th, m0, v0, g, t, HP)
    b1, b2 = HP.beta1, HP.beta2
    g64 = g.astype(np.float64)
    em = 4 * U * (np.abs(b1 * m0) + np.abs((1 - b1) * g64))
    ev = 6 * U * (np.abs(b2 * v0) + np.abs((1 - b2) * g64 * g64))
    assert (np.abs(m - rm) <= em).all()
    assert (np.abs(v - rv) <= ev).all()
    bc1, bc2 = 1 - b1 ** t, 1 - b2 ** t
    d = np.sqrt(rv / bc2) + HP.eps
    step = HP.lr / bc1 * rm / d
    awd = (1 - HP.lr * HP.weight_decay) * th.astype(np.float64)
    eth = 4 * U * np.abs(awd) + (HP.lr / bc1) * em / d + 12 * U * np.abs(step) + U * np.abs(rt)
    err = np.abs(master - rt)
    assert (err <= eth).all(), float((err / eth).max())


def test_adamw_ten_steps_vs_torch_normwise():
    """flat1m-style: N_d = 1, 10 steps from m = v = 0 against torch.optim.AdamW
    in float64 fed the same per-step averaged gradients."""
    rng = np.random.default_rng(7)
    n = 1 << 18
    th = (rng.standard_normal(n) * 0.02).astype(np.float32)
    master, m, v = th.copy(), np.zeros(n, np.float32), np.zeros(n, np.float32)
    p64 = torch.nn.Parameter(torch.from_numpy(th.astype(np.float64)))
    opt = torch.optim.AdamW([p64], lr=HP.lr, betas=(HP.beta1, HP.beta2), eps=HP.eps,
                            weight_decay=HP.weight_decay, foreach=False)
    for t in range(1, 11):
        gb = bf16_of((rng.standard_normal(n) * 1e-3).astype(np.float32))
        oracle.shard_step([gb], master, m, v, HP, t)
        p64.grad = torch.from_numpy(oracle.widen_bf16(gb).astype(np.float64))
        opt.step()
    st = opt.state[p64]

    def rel(a, b):
        return np.linalg.norm(a - b) / np.linalg.norm(b)

    assert rel(master, p64.detach().numpy()) < 1e-6
    assert rel(m, st["exp_avg"].numpy()) < 1e-6
    assert rel(v, st["exp_avg_sq"].numpy()) < 2e-6


def test_sharded_equals_unsharded():
    """AdamW is element-wise: concatenating every rank's shard update equals
    the update of the whole padded flat buffer, bitwise."""
    rng = np.random.default_rng(8)
    numel = [37, 5, 0, 64, 19, 11]
    for cap, n_d in ((0, 4), (24, 4), (31, 3), (16, 8)):
        pl = oracle.plan(numel, cap, n_d)
        ranks = []
        for q in range(n_d):
            ts = [bf16_of((rng.standard_normal(k) * 1e-3).astype(np.float32)) for k in numel]
            ranks.append(oracle.pack(ts, pl))
        th = (rng.standard_normal(pl.padded_total) * 0.02).astype(np.float32)
        # zero the pads of the state, as a real flat parameter would have them
        pad_mask = np.ones(pl.padded_total, bool)
        for r in range(n_d):
            f, s = pl.map(r, np.arange(pl.shard_len))
            pad_mask[f[s >= 0]] = False
        th[pad_mask] = 0
        full = _step(ranks, pl.padded_total, 3, master=th.copy())
        got = [np.empty_like(a) for a in full]
        for r in range(n_d):
            f, _ = pl.map(r, np.arange(pl.shard_len))
            sh = _step([oracle.slice_shard(x, pl, r) for x in ranks], pl.shard_len, 3,
                       master=th[f].copy())
            for dst, src in zip(got, sh):
                dst[f] = src
        for a, b in zip(full, got):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
        # pads stay +0 in every output
        for a in full[:4]:
            assert not a[pad_mask].view(np.uint8).any()


# ------------------------------------------------------------------ memory formulas
@pytest.mark.parametrize("name", workloads.NAMES)
def test_memory_formulas(name):
    """Per-GPU model-state bytes of the buffers each mode holds equal the
    page's closed forms with k = 12 and Psi -> P (padded), N_d = P / S."""
    w = workloads.get(name)
    pl = oracle.plan(w.numel, w.cap, w.n_d)
    P, S, N = pl.padded_total, pl.shard_len, w.n_d
    k = 12
    assert P == N * S
    assert oracle.model_state_bytes("baseline", P, S) == 2 * P + 2 * P + k * P
    assert oracle.model_state_bytes("zero1", P, S) == 2 * P + 2 * P + k * P / N
    assert oracle.model_state_bytes("zero2", P, S) == 2 * P + (2 * P + k * P) / N
    assert oracle.model_state_bytes("zero3", P, S) == (2 * P + 2 * P + k * P) / N



# ------------------------------------------------------------------ communication volumes
def _ring_reduce_scatter(bufs):
    """A ring Reduce-Scatter played step by step: every rank's buffer is cut
    into N chunks; in step s, rank r sends its running copy of chunk
    (r - s) mod N to rank r + 1, which adds it to its own copy.  Returns, per
    rank, (the chunk it ends with, that chunk's index) and the bytes each rank
    sent with 2-byte elements."""
    n = len(bufs)
    c = len(bufs[0]) // n
    cur = [[list(b[k * c:(k + 1) * c]) for k in range(n)] for b in bufs]
    sent = [0] * n
    for s in range(n - 1):
        msgs = [(r, (r - s) % n, list(cur[r][(r - s) % n])) for r in range(n)]
        for r, k, data in msgs:
            sent[r] += 2 * len(data)
            dst = (r + 1) % n
            cur[dst][k] = [a + b for a, b in zip(cur[dst][k], data)]
    return [(cur[r][(r + 1) % n], (r + 1) % n) for r in range(n)], sent


def _ring_all_gather(owned):
    """A ring All-Gather played step by step: rank r starts with chunk
    owned[r] = (data, index); in step s it forwards the chunk it received in
    step s - 1 (its own in step 0) to rank r + 1.  Returns every rank's
    assembled buffer and the bytes each rank sent with 2-byte elements."""
    n = len(owned)
    have = [{k: list(d)} for d, k in owned]
    last = [k for _, k in owned]
    sent = [0] * n
    for _ in range(n - 1):
        msgs = [(r, last[r], have[r][last[r]]) for r in range(n)]
        for r, k, data in msgs:
            sent[r] += 2 * len(data)
            dst = (r + 1) % n
            have[dst][k] = list(data)
            last[dst] = k
    full = [[x for k in range(n) for x in have[r][k]] for r in range(n)]
    return full, sent


@pytest.mark.parametrize("n_d", [1, 2, 3, 4, 5, 8])
def test_comm_volume_ring_simulation(n_d):
    """Bytes one GPU sends per step equal those of a played-out ring: naive
    DP All-Reduces the gradients (Reduce-Scatter + All-Gather), ZeRO-1/2
    Reduce-Scatter the gradients and All-Gather the updated parameters,
    ZeRO-3 All-Gathers the parameters twice (forward, backward) and
    Reduce-Scatters the gradients.  The played ring also has to compute the
    right results."""
    rng = np.random.default_rng(n_d)
    P = n_d * 6
    bufs = [rng.integers(-50, 50, P).tolist() for _ in range(n_d)]
    total = [sum(b[i] for b in bufs) for i in range(P)]
    c = P // n_d
    reduced, sent_rs = _ring_reduce_scatter(bufs)
    assert sorted(k for _, k in reduced) == list(range(n_d))
    for chunk, k in reduced:
        assert chunk == total[k * c:(k + 1) * c]
    full, sent_ag = _ring_all_gather(reduced)
    assert all(f == total for f in full)
    assert len(set(sent_rs)) == 1 and len(set(sent_ag)) == 1
    rs, ag = sent_rs[0], sent_ag[0]
    assert oracle.comm_bytes_per_gpu("ddp", P, n_d) == rs + ag
    assert oracle.comm_bytes_per_gpu("zero1", P, n_d) == rs + ag
    assert oracle.comm_bytes_per_gpu("zero2", P, n_d) == rs + ag
    assert oracle.comm_bytes_per_gpu("zero3", P, n_d) == rs + 2 * ag


@pytest.mark.parametrize("name", workloads.NAMES)
def test_comm_volume_closed_forms(name):
    """Dropping the (N_d - 1) / N_d factor gives the page's 4 Psi (naive DP,
    ZeRO-1, ZeRO-2) and 6 Psi (ZeRO-3), with Psi -> P (padded)."""
    w = workloads.get(name)
    P = oracle.plan(w.numel, w.cap, w.n_d).padded_total
    f = w.n_d / (w.n_d - 1)
    for mode, k in (("ddp", 4), ("zero1", 4), ("zero2", 4), ("zero3", 6)):
        assert oracle.comm_bytes_per_gpu(mode, P, w.n_d) * f == pytest.approx(k * P, rel=1e-12)
