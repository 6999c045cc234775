"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

Bars (the update's stated tolerances): reduced gradients bit-exact; fp32
master / m / v within 1e-6 relative; bf16 parameters within 1 ulp.  The
kernels follow the oracle's operation order, so every comparison then also
asserts that each output is bit-identical (NaN payloads aside).
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_step_amd as z
import oracle
import synth
from synth import workloads

from gpu_cases import (CANARY, DEV, Case, assert_bf16_close, assert_bitwise, assert_f32_close,
                       sample_indices, u16)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_smoke_entry():
    import __graft_entry__
    __graft_entry__.smoke()


# ------------------------------------------------------------------ workloads
def run_steps(case: Case, full_check_steps=()):
    w = case.w
    case.init_state_gpu()
    case.init_state_oracle()
    for k in range(w.n_steps):
        t = w.t_first + k
        say(f"  {w.name}: step t={t}")
        grads = case.grads_gpu(t)
        case.step_gpu(t, grads)
        del grads
        case.step_oracle(t, case.grads_oracle(t))
        torch.cuda.synchronize()
        if k + 1 == w.n_steps or t in full_check_steps:
            stats = case.compare(f"{w.name} t={t}")
            say(f"  {w.name} t={t}: exact matches {stats} of {case.o_g.size}")
    case.check_canaries()
    return stats


def test_flat1m_ten_steps_bit_exact():
    """Flat 1,048,576-parameter shard, N_d = 4, rank 3, 10 steps; every shard
    element compared after every step, bit for bit."""
    case = Case(workloads.get("flat1m"))
    case.init_state_gpu()
    case.init_state_oracle()
    w = case.w
    for t in range(1, 11):
        case.step_gpu(t, case.grads_gpu(t))
        case.step_oracle(t, case.grads_oracle(t))
        torch.cuda.synchronize()
        case.compare(f"t={t}")
        assert_bitwise(case.master.cpu().numpy(), case.o_master, "master")
        assert_bitwise(case.m.cpu().numpy(), case.o_m, "exp_avg")
        assert_bitwise(case.v.cpu().numpy(), case.o_v, "exp_avg_sq")
        assert_bitwise(u16(case.pout)[case.flat_pos], case.o_p, "param")
    case.check_canaries(n_probe=1 << 22)
    assert w.n_steps == 10


def test_gpt2s_pack_matches_oracle():
    """GPT-2-small list, 25 MiB buckets, N_d = 8: one rank's packed padded
    flat buffer equals the oracle's pack of the same per-tensor grads."""
    w = workloads.get("gpt2s")
    case = Case(w, sample_idx=np.arange(8))
    tsegs = synth.tensor_segments(w.numel)
    key = synth.key(w.name, "grad", 2, 0, 1)
    tens = [torch.empty(n, dtype=torch.int16, device=DEV) for n in w.numel]
    for t, n in enumerate(w.numel):
        synth.fill_device(tens[t], tsegs[t], key, *w.grad)
    flat = torch.full((case.P,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_bucket_pack(case.L, tens, flat)
    torch.cuda.synchronize()
    host_t = [u16(t) for t in tens]
    exp = oracle.pack(host_t, case.pl)
    assert_bitwise(u16(flat), exp, "packed flat buffer")


@pytest.mark.timeout(300)
def test_pack_cuts_pieces_longer_than_2_pow_30():
    """A 3-element tensor, then one of 2^30 + 4103 elements in the same
    bucket (the pack cuts pieces at 2^30 elements, keeping the 16-byte
    phase), and the bucket's padding at N_d = 8.  The long tensor starts 6
    bytes into a 16-byte line of the flat buffer; its source is placed at the
    same phase (vector pieces with a 5-element head) or at another one
    (element-wise pieces).  The flat buffer equals the tensors in order,
    padding +0."""
    n0 = (1 << 30) + 4103
    L = z.Layout([3, n0], 0, 8, 3)
    P = L.padded
    head = torch.tensor([7, -9, 11], dtype=torch.int16, device=DEV)
    for off in (3, 1):
        src = torch.empty(n0 + 16, dtype=torch.int16, device=DEV)[off:off + n0]
        src.copy_(torch.arange(n0, dtype=torch.int32, device=DEV).to(torch.int16))
        flat = torch.full((P,), CANARY, dtype=torch.int16, device=DEV)
        z.zero_bucket_pack(L, [head, src], flat)
        torch.cuda.synchronize()
        assert torch.equal(flat[:3], head)
        assert torch.equal(flat[3:3 + n0], src), f"long tensor (source offset {off})"
        assert not flat[3 + n0:].any(), "bucket padding is +0"
        del src, flat
        torch.cuda.empty_cache()


@pytest.mark.timeout(300)
def test_pack_and_gather_split_into_several_launches():
    """One tensor of 2^32 + 12349 elements at N_d = 4 (one bucket, 3 pad
    elements): the pack needs 2^20 + 5 tiles of 4096 elements and the gather
    2^21 + 8 items of 2048 elements, more blocks than one launch takes (the
    dispatch grid counts work-items in 32 bits), so both are cut into several
    launches.  Pack: the flat buffer is the tensor, then +0 padding; gather
    of the flat buffer's four quarters (the rank shards): the flat buffer.
    Values are random 16-bit patterns, so a misplaced block shows."""
    n = (1 << 32) + 12349
    L = z.Layout([n], 0, 4, 2)
    P, S = L.padded, L.shard
    assert (P, S) == (n + 3, (n + 3) // 4) and S % 8 == 0
    gen = torch.Generator(device=DEV)
    gen.manual_seed(20260)
    src = torch.randint(-32768, 32768, (n,), dtype=torch.int16, device=DEV, generator=gen)
    flat = torch.full((P,), CANARY, dtype=torch.int16, device=DEV)
    say(f"  pack of {n} elements into {P}")
    z.zero_bucket_pack(L, [src], flat)
    torch.cuda.synchronize()
    assert torch.equal(flat[:n], src), "packed tensor"
    assert not flat[n:].any(), "bucket padding is +0"
    del src
    torch.cuda.empty_cache()
    shards = [flat[q * S:(q + 1) * S].clone() for q in range(4)]
    out = torch.full((P,), CANARY, dtype=torch.int16, device=DEV)
    say(f"  gather of 4 shards of {S} elements")
    z.zero_gather_params(L, shards, out)
    torch.cuda.synchronize()
    assert torch.equal(out, flat), "gathered flat buffer"
    del shards, out, flat
    torch.cuda.empty_cache()


def test_gpt2s_ten_steps_full():
    case = Case(workloads.get("gpt2s"))
    run_steps(case, full_check_steps=(1,))


@pytest.mark.timeout(900)
def test_llama8b_sampled():
    """Llama-3-8B list, 613 buckets of 25 MiB, N_d = 8, rank 7 (1.0e9-element
    shard, 16 GB of bf16 contributions), 10 steps from m = v = 0; sampled."""
    w = workloads.get("llama8b")
    case = Case(w, sample_idx=np.arange(1))
    case.__init__(w, sample_idx=sample_indices(case.S, case.pl))
    stats = run_steps(case)
    assert stats["param"] == case.idx.size


# ------------------------------------------------------------------ edge cases
@pytest.mark.timeout(600)
def test_shard_beyond_2_pow_31_elements_sampled():
    """A shard of 2^31 + 4099 elements (64-bit indexing everywhere; ragged
    tail), N_d = 2, rank 1, All-Gather slot output 2^32 + 8198 elements
    away from the start: sampled against the oracle."""
    S = (1 << 31) + 4099
    w = workloads.Workload("flat1m", [2 * S], 0, 2, 1, "compact", "ag_slot", 7, 1,
                           ("normal", 1e-3), ("normal", 0.02), ("normal", 1e-4),
                           ("absnormal", 1e-6))
    case = Case(w, sample_idx=np.arange(1))
    assert case.S == S
    idx = np.concatenate([sample_indices(S, case.pl, n_random=1 << 16),
                          np.arange((1 << 31) - 64, (1 << 31) + 64)])
    case.__init__(w, sample_idx=idx)
    stats = run_steps(case)
    assert stats["param"] == case.idx.size


@pytest.mark.timeout(300)
def test_accumulate_beyond_2_pow_31_elements_sampled():
    """no_sync accumulation over 2^31 + 5 elements (overwrite, add, then add
    with bf16 emit and no fp32 store), sampled against the oracle."""
    n = (1 << 31) + 5
    segs = [(0, 0, n, 0)]
    acc = torch.empty(n, dtype=torch.float32, device=DEV)
    g = torch.empty(n, dtype=torch.int16, device=DEV)
    emit = torch.empty(n, dtype=torch.int16, device=DEV)
    rng = np.random.default_rng(3)
    xs = np.unique(np.concatenate([rng.integers(0, n, 1 << 16), np.arange(n - 64, n),
                                   np.arange((1 << 31) - 64, (1 << 31) + 5)]))
    o_acc = np.zeros(xs.size, np.float32)
    for k, flags in enumerate((z.ACC_OVERWRITE, 0, z.ACC_EMIT_BF16 | z.ACC_NO_STORE)):
        key = synth.key("accum1p3b", "micro_grad", 0, k, 1)
        synth.fill_device(g, segs, key, "normal", 2e-3)
        z.zero_grad_accumulate(acc, g, 0.25, flags, emit if flags & z.ACC_EMIT_BF16 else None)
        o_out = oracle.accumulate(o_acc, synth.values_at(xs, key, "normal", 2e-3, synth.OUT_BF16),
                                  0.25, overwrite=(k == 0), store_acc=(k < 2), emit=(k == 2))
    torch.cuda.synchronize()
    sel = torch.from_numpy(xs).to(DEV)
    assert_bitwise(acc[sel].cpu().numpy(), o_acc, "accumulator")
    assert_bitwise(emit[sel].cpu().numpy().view(np.uint16), o_out, "emitted bf16")


EDGE = [
    # numel, cap, n_d, rank, grad_layout, out_mode
    ([1000, 37, 4096, 3], 1500, 4, 3, "flat", "ag_slot"),
    ([1000, 37, 4096, 3], 1500, 4, 0, "compact", "shard"),
    ([17], 0, 1, 0, "flat", "ag_slot"),                     # N_d = 1: no reduction
    ([5, 0, 123, 64], 40, 3, 2, "flat", "ag_slot"),         # non-power-of-two N_d, empty tensor
    ([999, 1001], 0, 5, 4, "compact", "ag_slot"),
    ([4096 * 7 + 5], 4096, 7, 6, "flat", "shard"),
    ([70000, 3], 16384, 8, 7, "flat", "ag_slot"),           # ragged last bucket (slice % 8 != 0)
    ([50000], 8008, 8, 3, "flat", "ag_slot"),               # slice 1001: unaligned flat slots
    ([50000], 8032, 8, 3, "flat", "ag_slot"),               # slice 1004: 4- but not 8-aligned
    ([4 * 2503], 0, 4, 1, "compact", "shard"),              # 2503: 4 full chunks + 455 tail
    ([20 * 1040 + 12], 1040, 4, 2, "flat", "ag_slot"),      # slice 260: chunks cross buckets
    ([20000, 20001], 0, 16, 15, "compact", "ag_slot"),
    ([65536 + 13], 0, 32, 31, "flat", "ag_slot"),
    ([64 * 300 + 1], 6400, 64, 63, "compact", "shard"),     # N_d = 64 with padded tails
    ([64 * 300 + 1], 6400, 64, 0, "flat", "ag_slot"),
    # N_d = 64 runs chunks of 1024 elements per wave: slices of 1040 make the
    # chunks cross bucket cuts, a 2-element last slice runs element-wise
    ([64 * 1040 * 6 + 70], 64 * 1040, 64, 63, "flat", "ag_slot"),
    ([64 * 1040 * 6 + 70], 64 * 1040, 64, 5, "compact", "ag_slot"),
    ([64 * 5003], 0, 64, 17, "compact", "shard"),         # 4 full chunks + 907 tail
    ([100 * 97], 0, 100, 99, "compact", "shard"),           # generic rank count
    ([256 * 33 + 7], 0, 256, 255, "flat", "ag_slot"),       # largest rank count
    ([8], 0, 8, 5, "flat", "ag_slot"),                      # one element per rank
    ([3], 0, 8, 7, "flat", "ag_slot"),                      # this rank holds only padding
    # N_d = 2: five vector buckets, then a last slot at an odd flat offset
    ([2 * 4096 * 3 + 999, 77], 5000, 2, 1, "flat", "ag_slot"),
    ([2 * 70000 + 1], 0, 2, 0, "compact", "shard"),         # 136 full chunks + 369 tail
    # N_d = 32: slices of 1040, a 2-element last slice
    ([32 * 1040 * 3 + 45], 32 * 1040, 32, 7, "compact", "ag_slot"),
]


def _edge_case(numel, cap, n_d, rank, gl, om, t=3, rows=None):
    w = workloads.Workload("edge", numel, cap, n_d, rank, gl, om, t, 1, ("normal", 1e-3),
                           ("normal", 0.02), ("normal", 1e-4), ("absnormal", 1e-6), rows=rows)
    w.name = "flat1m"  # reuse a workload id for the generator keys
    return Case(w)


@pytest.mark.parametrize("numel,cap,n_d,rank,gl,om", EDGE)
def test_edge_cases_full_compare(numel, cap, n_d, rank, gl, om):
    case = _edge_case(numel, cap, n_d, rank, gl, om)
    say(f"  edge numel={numel} cap={cap} n_d={n_d} r={rank} {gl} {om}: S={case.S}")
    case.init_state_gpu()
    case.init_state_oracle()
    for t in (1, 2, 3):
        case.step_gpu(t, case.grads_gpu(t))
        case.step_oracle(t, case.grads_oracle(t))
    torch.cuda.synchronize()
    case.compare("edge")
    for a, b in ((case.master, case.o_master), (case.m, case.o_m), (case.v, case.o_v)):
        assert_bitwise(a.cpu().numpy(), b, "state")
    pos = case.flat_pos if om == "ag_slot" else np.arange(case.S)
    assert_bitwise(u16(case.pout)[pos], case.o_p, "param")
    case.check_canaries(n_probe=4096)


@pytest.mark.parametrize("gl,om", [("flat", "ag_slot"), ("compact", "shard")])
def test_planned_placement_gives_identical_results(gl, om):
    """The step on buffers carved from one pool laid out by
    zero_placement_plan (lanes of 1 MiB here, so the lane structure is
    exercised at a small size) equals the step on separate allocations."""
    from fsdp_sharded_optimizer_step_amd import placement as zp
    case = _edge_case([300_001, 77], 65_536, 8, 5, gl, om)
    case.init_state_gpu()
    grads = case.grads_gpu(2)
    # the shift is chosen by a timing callback; this one makes the last of
    # the three candidate shifts (0, 1, 2 MiB) the fastest
    times = iter([3.0, 2.0, 1.0])
    pool = zp.step_pool(case.L, grad_layout=z.GRAD_FLAT if gl == "flat" else z.GRAD_COMPACT,
                        out_mode=z.OUT_AG_SLOT if om == "ag_slot" else z.OUT_SHARD,
                        reduced_grad=True, lane_bytes=1 << 20, n_lanes=3, align=256,
                        slack=2 << 20, choose=lambda views: next(times), shift_step=1 << 20)
    assert [sh for sh, _ in pool.tuning] == [0, 1 << 20, 2 << 20] and pool.shift == 2 << 20
    assert len({(o - pool.shift) // (1 << 20) % 3 for o in pool.offsets.values()}) == 3
    assert pool["master"].data_ptr() == pool.buf.data_ptr() + pool.offsets["master"]
    for q, g in enumerate(grads):
        pool[f"g{q}"].copy_(g)
    for name, t in (("master", case.master), ("exp_avg", case.m), ("exp_avg_sq", case.v),
                    ("param_out", case.pout)):
        pool[name].copy_(t)
    case.step_gpu(2, grads)
    z.zero_shard_step(case.L, case.hp_z, 2, [pool[f"g{q}"] for q in range(8)],
                      z.GRAD_FLAT if gl == "flat" else z.GRAD_COMPACT, pool["master"],
                      pool["exp_avg"], pool["exp_avg_sq"], pool["param_out"],
                      z.OUT_AG_SLOT if om == "ag_slot" else z.OUT_SHARD, pool["reduced_grad"])
    torch.cuda.synchronize()
    for name, t in (("master", case.master), ("exp_avg", case.m), ("exp_avg_sq", case.v),
                    ("param_out", case.pout), ("reduced_grad", case.gout)):
        assert torch.equal(pool[name].cpu(), t.cpu()), name


def test_tuned_step_pool_times_the_step_at_each_shift():
    from fsdp_sharded_optimizer_step_amd import placement as zp
    L = z.Layout([300_001, 77], 65_536, 8, 5)
    pool = zp.tuned_step_pool(L, z.AdamW(), 1, z.GRAD_COMPACT, z.OUT_SHARD, slack=2 << 20,
                              lane_bytes=1 << 20, align=256, shift_step=1 << 20)
    assert [sh for sh, _ in pool.tuning] == [0, 1 << 20, 2 << 20]
    assert all(ms > 0 for _, ms in pool.tuning)
    assert pool.shift == min(pool.tuning, key=lambda x: x[1])[0]
    assert len(pool.grads) == 8 and pool["param_out"].numel() == L.shard


def test_tuned_step_pool_times_the_call_its_buffers_are_for(monkeypatch):
    """A pool holding fp32 accumulators is placed by timing the fused step
    (zero_shard_step_accumulate) on them, with the reduced gradient written
    when the pool holds one."""
    from fsdp_sharded_optimizer_step_amd import placement as zp
    calls = []
    real = zp.zero_shard_step_accumulate

    def spy(layout, hp, t, acc, micro, *a):
        calls.append((len(acc), len(micro), a[-1] is not None))
        return real(layout, hp, t, acc, micro, *a)

    monkeypatch.setattr(zp, "zero_shard_step_accumulate", spy)
    L = z.Layout([300_001, 77], 65_536, 4, 3)
    pool = zp.tuned_step_pool(L, z.AdamW(), 1, z.GRAD_COMPACT, z.OUT_SHARD, slack=2 << 20,
                              lane_bytes=1 << 20, align=256, shift_step=1 << 20,
                              accumulators=True, reduced_grad=True)
    assert len(pool.tuning) == 3 and calls
    assert all(c == (4, 4, True) for c in calls)


def test_tuned_step_pool_falls_back_to_a_search_that_fits(monkeypatch):
    """With no explicit slack the helper tries its searches in order: one
    whose pool cannot be allocated is skipped for the next."""
    from fsdp_sharded_optimizer_step_amd import placement as zp
    monkeypatch.setattr(zp, "SEARCH", ((1 << 50, 1 << 20), (2 << 20, 1 << 20)))
    L = z.Layout([300_001, 77], 65_536, 8, 5)
    pool = zp.tuned_step_pool(L, z.AdamW(), 1, z.GRAD_COMPACT, z.OUT_SHARD,
                              lane_bytes=1 << 20, align=256)
    assert [sh for sh, _ in pool.tuning] == [0, 1 << 20, 2 << 20]
    assert pool.shift == min(pool.tuning, key=lambda x: x[1])[0]
    with pytest.raises(TypeError):
        zp.tuned_step_pool(L, z.AdamW(), 1, shift_step=1 << 20)


def test_empty_shard_is_a_no_op():
    L = z.Layout([], 0, 4, 0)
    e = torch.empty(0, dtype=torch.float32, device=DEV)
    h = torch.empty(0, dtype=torch.int16, device=DEV)
    z.zero_shard_step(L, z.AdamW(), 1, [h] * 4, z.GRAD_COMPACT, e, e.clone(), e.clone(), h.clone(),
                      z.OUT_SHARD)
    torch.cuda.synchronize()


def test_all_ranks_assemble_the_unsharded_update():
    """Every rank steps its own shard into its All-Gather slot of one shared
    buffer; the assembled buffer and states equal the oracle's update of the
    whole padded flat buffer (sharded == unsharded)."""
    numel, cap, n_d, t = [301, 77, 1024, 5, 900], 640, 4, 2
    pl = oracle.plan(numel, cap, n_d)
    P = pl.padded_total
    rng = np.random.default_rng(9)
    flats_h = []
    for q in range(n_d):
        ts = [synth.fill_host(n, synth.OUT_BF16, [(0, sum(numel[:k]), n, 0)],
                              synth.key("gpt2s", "grad", q, 0, t), "normal", 1e-3)
              for k, n in enumerate(numel)]
        flats_h.append(oracle.pack(ts, pl))
    th = (rng.standard_normal(P) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(P) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(P) * 1e-6).astype(np.float32)
    pads = np.ones(P, bool)
    for r in range(n_d):
        f, s = pl.map(r, np.arange(pl.shard_len))
        pads[f[s >= 0]] = False
    th[pads] = 0
    m0[pads] = 0
    v0[pads] = 0
    full = [th.copy(), m0.copy(), v0.copy()]
    p_full, _ = oracle.shard_step(flats_h, *full, oracle.AdamW(), t)
    flats = [torch.from_numpy(f.view(np.int16)).to(DEV) for f in flats_h]
    ag = torch.full((P,), CANARY, dtype=torch.int16, device=DEV)
    got = [np.zeros(P, np.float32) for _ in range(3)]
    for r in range(n_d):
        L = z.Layout(numel, cap, n_d, r)
        f, _ = pl.map(r, np.arange(pl.shard_len))
        st = [torch.from_numpy(a[f].copy()).to(DEV) for a in (th, m0, v0)]
        z.zero_shard_step(L, z.AdamW(), t, flats, z.GRAD_FLAT, *st, ag, z.OUT_AG_SLOT)
        torch.cuda.synchronize()
        for dst, src in zip(got, st):
            dst[f] = src.cpu().numpy()
    assert_bitwise(u16(ag), p_full, "assembled All-Gather buffer")
    for a, b in zip(got, full):
        assert_bitwise(a, b, "assembled state")


@pytest.mark.parametrize("launch", [(1, 64, 0), (7, 192, 0), (64, 256, 0), (3000, 128, 0),
                                    (0, 0, 1), (5, 64, 1), (100000, 256, 0)])
def test_launch_shape_invariance(launch):
    """Results are bit-identical for any grid / block size and for the scalar
    path (no reduction across lanes, fixed rank order)."""
    numel, cap, n_d, rank = [300_000, 12_345, 777], 65_536, 8, 6
    outs = []
    for lc in (None, launch):
        case = _edge_case(numel, cap, n_d, rank, "flat", "ag_slot")
        case.init_state_gpu()
        grads = case.grads_gpu(5)
        case.step_gpu(5, grads, launch=lc)
        torch.cuda.synchronize()
        outs.append([case.master.cpu().numpy(), case.m.cpu().numpy(), case.v.cpu().numpy(),
                     u16(case.pout), case.gout.cpu().numpy()])
    for a, b in zip(*outs):
        assert_bitwise(a, b, f"launch {launch}")


@pytest.mark.parametrize("launch", [(1, 64, 0), (13, 192, 0), (3000, 128, 0), (0, 0, 1)])
def test_launch_shape_invariance_at_64_ranks(launch):
    """The same at N_d = 64, whose vector kernel takes 1024-element chunks
    per wave: bit-identical for any grid / block size and the scalar path."""
    numel, cap, n_d, rank = [64 * 1040 * 9 + 200, 64 * 77], 64 * 1040, 64, 62
    outs = []
    for lc in (None, launch):
        case = _edge_case(numel, cap, n_d, rank, "flat", "ag_slot")
        case.init_state_gpu()
        grads = case.grads_gpu(4)
        case.step_gpu(4, grads, launch=lc)
        torch.cuda.synchronize()
        outs.append([case.master.cpu().numpy(), case.m.cpu().numpy(), case.v.cpu().numpy(),
                     u16(case.pout), case.gout.cpu().numpy()])
    for a, b in zip(*outs):
        assert_bitwise(a, b, f"launch {launch}")


def test_misaligned_buffers_take_the_scalar_path():
    """Buffers offset by one element (2 or 4 bytes from 16-byte alignment)
    give the same results as the oracle."""
    numel, n_d, t = [5000], 4, 2
    pl = oracle.plan(numel, 0, n_d)
    S = pl.shard_len
    rng = np.random.default_rng(11)
    gh = [(rng.standard_normal(S) * 1e-3).astype(np.float32) for _ in range(n_d)]
    gh = [oracle.round_bf16(g) for g in gh]
    th = (rng.standard_normal(S) * 0.02).astype(np.float32)
    m0 = (rng.standard_normal(S) * 1e-4).astype(np.float32)
    v0 = np.abs(rng.standard_normal(S) * 1e-6).astype(np.float32)

    def off(a, dt):
        buf = torch.empty(a.size + 1, dtype=dt, device=DEV)
        view = buf[1:]
        view.copy_(torch.from_numpy(a.view(np.int16) if dt == torch.int16 else a))
        return view

    L = z.Layout(numel, 0, n_d, 1)
    grads = [off(g, torch.int16) for g in gh]
    st = [off(a.copy(), torch.float32) for a in (th, m0, v0)]
    p = torch.empty(S + 1, dtype=torch.int16, device=DEV)[1:]
    z.zero_shard_step(L, z.AdamW(), t, grads, z.GRAD_COMPACT, *st, p, z.OUT_SHARD)
    torch.cuda.synchronize()
    o = [th.copy(), m0.copy(), v0.copy()]
    ep, _ = oracle.shard_step(gh, *o, oracle.AdamW(), t)
    for a, b in zip(st, o):
        assert_bitwise(a.cpu().numpy(), b, "state")
    assert_bitwise(u16(p), ep, "param")


def test_nonfinite_gradients_propagate_elementwise():
    n_d, S, t = 4, 4096, 1
    rng = np.random.default_rng(12)
    gh = [oracle.round_bf16((rng.standard_normal(S) * 1e-3).astype(np.float32))
          for _ in range(n_d)]
    gh[2][100] = 0x7F80   # +inf
    gh[1][200] = 0xFFC1   # NaN
    gh[0][300] = 0x7F80
    gh[3][300] = 0xFF80   # inf - inf = NaN
    th = (rng.standard_normal(S) * 0.02).astype(np.float32)
    L = z.Layout([S * n_d], 0, n_d, 0)
    grads = [torch.from_numpy(g.view(np.int16)).to(DEV) for g in gh]
    st = [torch.from_numpy(a).to(DEV) for a in (th.copy(), np.zeros(S, np.float32),
                                                 np.zeros(S, np.float32))]
    p = torch.empty(S, dtype=torch.int16, device=DEV)
    gout = torch.empty(S, dtype=torch.float32, device=DEV)
    z.zero_shard_step(L, z.AdamW(), t, grads, z.GRAD_COMPACT, *st, p, z.OUT_SHARD, gout)
    torch.cuda.synchronize()
    o = [th.copy(), np.zeros(S, np.float32), np.zeros(S, np.float32)]
    ep, eg = oracle.shard_step(gh, *o, oracle.AdamW(), t, want_grad=True)
    gm = st[0].cpu().numpy()
    bad = np.isnan(gm) | np.isinf(gm)
    assert set(np.flatnonzero(bad)) <= {100, 200, 300}
    ok = np.ones(S, bool)
    ok[[100, 200, 300]] = False
    assert_bitwise(gm[ok], o[0][ok], "finite elements")
    assert np.isnan(gout.cpu().numpy()[[200, 300]]).all()
    assert np.isinf(gout.cpu().numpy()[100])
    assert_bitwise(u16(p)[ok], ep[ok], "finite params")


@pytest.mark.parametrize("contrib", ["bf16", "f32", "fused"])
def test_subnormals_are_kept_bitwise(contrib):
    """Subnormal contributions, moments, master weights and sums: the kernels
    keep IEEE subnormals (no flush to zero), as the oracle does; every output
    is compared bit for bit, three steps (t = 1 makes v' = C2*g*g subnormal)."""
    n_d, S = 8, 8192
    rng = np.random.default_rng(21)

    def sub32(n, lo=1, hi=0x007FFFFF):     # positive and negative binary32 subnormals
        b = rng.integers(lo, hi, n).astype(np.uint32) | (rng.integers(0, 2, n).astype(np.uint32) << 31)
        return b.view(np.float32)

    def mix32(n, scale):
        x = (rng.standard_normal(n) * scale).astype(np.float32)
        k = rng.random(n) < 0.5
        x[k] = sub32(int(k.sum()))
        return x

    L = z.Layout([S * n_d], 0, n_d, 3)
    th, m, v = mix32(S, 1e-38), mix32(S, 1e-38), np.abs(mix32(S, 1e-39))
    dev_state = [torch.from_numpy(a.copy()).to(DEV) for a in (th, m, v)]
    o_state = [a.copy() for a in (th, m, v)]
    p = torch.empty(S, dtype=torch.int16, device=DEV)
    gout = torch.empty(S, dtype=torch.float32, device=DEV)
    hp_z, hp_o = z.AdamW(lr=1e-38, eps=1e-40), oracle.AdamW(lr=1e-38, eps=1e-40)
    for t in (1, 2, 3):
        if contrib == "bf16":
            # bf16 subnormal patterns 0x0001..0x007F (and negatives), some normals
            gh = [np.where(rng.random(S) < 0.7, rng.integers(1, 0x80, S),
                           rng.integers(0x0080, 0x0400, S)).astype(np.uint16)
                  | (rng.integers(0, 2, S).astype(np.uint16) << 15) for _ in range(n_d)]
            z.zero_shard_step(L, hp_z, t, [torch.from_numpy(g.view(np.int16)).to(DEV)
                                           for g in gh], z.GRAD_COMPACT, *dev_state, p,
                              z.OUT_SHARD, gout)
            ep, eg = oracle.shard_step(gh, *o_state, hp_o, t, want_grad=True)
        else:
            acc = [mix32(S, 1e-38) for _ in range(n_d)]
            if contrib == "f32":
                z.zero_shard_step(L, hp_z, t, [torch.from_numpy(a).to(DEV) for a in acc],
                                  z.GRAD_COMPACT, *dev_state, p, z.OUT_SHARD, gout)
                ep, eg = oracle.shard_step_f32(acc, *o_state, hp_o, t, want_grad=True)
            else:
                mic = [(rng.integers(1, 0x80, S).astype(np.uint16)
                        | (rng.integers(0, 2, S).astype(np.uint16) << 15)) for _ in range(n_d)]
                z.zero_shard_step_accumulate(
                    L, hp_z, t, [torch.from_numpy(a).to(DEV) for a in acc],
                    [torch.from_numpy(g.view(np.int16)).to(DEV) for g in mic], 0.25,
                    z.DTYPE_BF16, z.GRAD_COMPACT, *dev_state, p, z.OUT_SHARD, gout)
                contribs = [oracle.accumulate(a.copy(), g, 0.25, overwrite=False,
                                              store_acc=False, emit=True)
                            for a, g in zip(acc, mic)]
                ep, eg = oracle.shard_step(contribs, *o_state, hp_o, t, want_grad=True)
        torch.cuda.synchronize()
        assert_bitwise(gout.cpu().numpy(), eg, f"{contrib} t={t} reduced gradient")
        for a, b, what in zip(dev_state, o_state, ("master", "m", "v")):
            assert_bitwise(a.cpu().numpy(), b, f"{contrib} t={t} {what}")
        assert_bitwise(u16(p), ep, f"{contrib} t={t} param")
    # the test is only meaningful if subnormals actually occurred
    for x in (eg, o_state[1], o_state[2]):
        x = np.asarray(x)
        assert ((x != 0) & (np.abs(x) < np.float32(1.1754944e-38))).any()


def test_repeat_calls_are_deterministic():
    outs = []
    for _ in range(2):
        case = _edge_case([123_457, 99], 50_000, 8, 3, "compact", "ag_slot")
        case.init_state_gpu()
        case.step_gpu(4, case.grads_gpu(4))
        torch.cuda.synchronize()
        outs.append([case.master.cpu().numpy(), u16(case.pout), case.gout.cpu().numpy()])
    for a, b in zip(*outs):
        assert_bitwise(a, b, "repeat")


def _hip_runtime():
    """The HIP runtime instance this process (and the library) uses."""
    import ctypes
    z.load()
    with open("/proc/self/maps") as f:
        paths = sorted({ln.split()[-1] for ln in f if "libamdhip64.so" in ln})
    assert paths, "libamdhip64 is not mapped"
    hip = ctypes.CDLL(paths[0])
    hip.hipMalloc.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_size_t]
    return hip


def test_pending_hip_error_refuses_the_call_before_any_launch():
    """A HIP error left pending by an earlier, unrelated call (here an
    impossible allocation, forced from the host) makes the step return
    ZERO_EHIP without enqueuing anything and without clearing that error;
    once the caller has read it, the same call runs and equals the oracle."""
    import ctypes
    hip = _hip_runtime()
    case = _edge_case([5000, 33], 1024, 4, 1, "compact", "ag_slot")
    case.init_state_gpu()
    case.init_state_oracle()
    grads = case.grads_gpu(3)
    torch.cuda.synchronize()
    before = [case.master.clone(), case.pout.clone()]
    p = ctypes.c_void_p()
    assert hip.hipMalloc(ctypes.byref(p), 1 << 62) != 0
    if hip.hipPeekAtLastError() == 0:
        pytest.skip("this HIP runtime does not keep a failed allocation as the last error")
    with pytest.raises(z.ZeroError) as e:
        case.step_gpu(3, grads)
    assert e.value.status == z.binding.ZERO_EHIP
    assert hip.hipGetLastError() != 0          # still pending for the caller; now cleared
    torch.cuda.synchronize()
    assert torch.equal(case.master, before[0]) and torch.equal(case.pout, before[1])
    case.step_gpu(3, grads)
    case.step_oracle(3, case.grads_oracle(3))
    torch.cuda.synchronize()
    case.compare("after the pending error was read")


# ------------------------------------------------------------------ accumulate
@pytest.mark.parametrize("n,offset", [(1 << 20, 0), ((1 << 20) + 5, 0), (1003, 1), (7, 0)])
def test_accumulate_modes_match_oracle(n, offset):
    rng = np.random.default_rng(13)
    g = [oracle.round_bf16((rng.standard_normal(n) * 2e-3).astype(np.float32)) for _ in range(4)]
    acc0 = rng.standard_normal(n).astype(np.float32)

    def dev(a, dt):
        buf = torch.empty(a.size + offset, dtype=dt, device=DEV)[offset:]
        buf.copy_(torch.from_numpy(a.view(np.int16) if dt == torch.int16 else a))
        return buf

    for flags in (z.ACC_OVERWRITE, 0, z.ACC_EMIT_BF16, z.ACC_EMIT_BF16 | z.ACC_NO_STORE,
                  z.ACC_OVERWRITE | z.ACC_EMIT_BF16,
                  z.ACC_OVERWRITE | z.ACC_EMIT_BF16 | z.ACC_NO_STORE):
        acc = dev(acc0.copy(), torch.float32)
        out = dev(np.zeros(n, np.uint16), torch.int16)
        gd = dev(g[1], torch.int16)
        z.zero_grad_accumulate(acc, gd, 0.25, flags, out if flags & z.ACC_EMIT_BF16 else None)
        torch.cuda.synchronize()
        o_acc = acc0.copy()
        emit = bool(flags & z.ACC_EMIT_BF16)
        o_out = oracle.accumulate(o_acc, g[1], 0.25, overwrite=bool(flags & z.ACC_OVERWRITE),
                                  store_acc=not (flags & z.ACC_NO_STORE), emit=emit)
        assert_bitwise(acc.cpu().numpy(), o_acc, f"acc flags={flags}")
        if emit:
            assert_bitwise(u16(out), o_out, f"bf16 flags={flags}")


def test_accumulate_four_micro_batches_equal_full_batch_mean_on_gpu():
    n = (1 << 18) + 3
    rng = np.random.default_rng(14)
    g = [oracle.round_bf16((rng.standard_normal(n) * 2e-3).astype(np.float32)) for _ in range(4)]
    acc = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    for k in range(4):
        z.zero_grad_accumulate(acc, torch.from_numpy(g[k].view(np.int16)).to(DEV), 0.25,
                               z.ACC_OVERWRITE if k == 0 else 0)
    torch.cuda.synchronize()
    w = [oracle.widen_bf16(x) for x in g]
    mean = (((w[0] + w[1]) + w[2]) + w[3]) / np.float32(4)
    assert_bitwise(acc.cpu().numpy(), mean, "accumulated mean")


# ------------------------------------------------------------------ cast
@pytest.mark.timeout(600)
def test_gpu_bf16_cast_exhaustive():
    """With lr = wd = 0, zero gradients and moments, the step leaves every
    master value unchanged and writes bf16(master): all 2^32 binary32
    patterns, compared with the oracle's rounding."""
    from concurrent.futures import ThreadPoolExecutor
    hp = z.AdamW(lr=0.0, weight_decay=0.0, eps=1.0)
    chunk = 1 << 28
    L = z.Layout([chunk], 0, 1, 0)
    g = torch.zeros(chunk, dtype=torch.int16, device=DEV)
    m = torch.zeros(chunk, dtype=torch.float32, device=DEV)
    v = torch.zeros_like(m)
    p = torch.empty(chunk, dtype=torch.int16, device=DEV)
    base = torch.arange(chunk, dtype=torch.int64, device=DEV)
    sub = chunk // 16
    with ThreadPoolExecutor(16) as ex:
        for c in range((1 << 32) // chunk):
            lo = c * chunk
            signed_lo = lo - (1 << 32) if lo >= (1 << 31) else lo
            th = (base + signed_lo).to(torch.int32).view(torch.float32).contiguous()
            m.zero_()
            v.zero_()
            z.zero_shard_step(L, hp, 1, [g], z.GRAD_COMPACT, th, m, v, p, z.OUT_SHARD)
            torch.cuda.synchronize()
            exp = np.concatenate(list(ex.map(
                lambda k: oracle.round_bf16_patterns(lo + k * sub, lo + (k + 1) * sub),
                range(16))))
            got = u16(p)
            pats = np.arange(lo, lo + chunk, dtype=np.uint64).astype(np.uint32)
            nan = ((pats & 0x7F800000) == 0x7F800000) & ((pats & 0x7FFFFF) != 0)
            assert_bitwise(got[~nan], exp[~nan], f"cast chunk {c}")
            gn = got[nan].astype(np.uint32)
            assert (((gn & 0x7F80) == 0x7F80) & ((gn & 0x7F) != 0)).all()
            say(f"  cast chunk {c} ok")


# ------------------------------------------------------------------ bucket ranges
BUCKET_RANGES = [
    # numel, cap, n_d, rank, grad_layout, out_mode
    ([70000, 3], 16384, 8, 7, "flat", "ag_slot"),           # ragged last bucket, unaligned
    ([1000, 37, 4096, 3], 1500, 4, 3, "flat", "ag_slot"),   # slices of 375: scalar path
    ([4096 * 7 + 5], 4096, 7, 6, "flat", "shard"),
    ([50000], 8008, 8, 3, "compact", "ag_slot"),
    ([20000, 20001], 4000, 16, 15, "compact", "shard"),
    ([64 * 300 + 1], 6400, 64, 63, "flat", "ag_slot"),
    ([8192 * 6], 8192, 8, 2, "flat", "ag_slot"),            # six equal buckets
    ([100 * 97], 1000, 100, 99, "compact", "shard"),         # runtime rank count
    ([64 * 1040 * 6 + 70], 64 * 1040, 64, 63, "flat", "ag_slot"),  # 1024-element chunks
]


def _step_buckets(case, t, grads, b0, b1):
    w = case.w
    gl = z.GRAD_FLAT if w.grad_layout == "flat" else z.GRAD_COMPACT
    om = z.OUT_AG_SLOT if w.out_mode == "ag_slot" else z.OUT_SHARD
    z.zero_shard_step_buckets(case.L, case.hp_z, t, b0, b1, grads, gl, case.master, case.m,
                              case.v, case.pout, om, case.gout)


def _random_ranges(nb, rng):
    cuts = sorted(set(int(c) for c in rng.integers(0, nb + 1, 4)) | {0, nb})
    ranges = list(zip(cuts[:-1], cuts[1:]))
    rng.shuffle(ranges)
    return ranges


@pytest.mark.parametrize("numel,cap,n_d,rank,gl,om", BUCKET_RANGES)
def test_bucket_ranges_in_any_order_equal_the_oracle(numel, cap, n_d, rank, gl, om):
    """Every bucket stepped once per step, in random groups and order, gives
    the oracle's whole-shard step bit for bit."""
    case = _edge_case(numel, cap, n_d, rank, gl, om)
    rng = np.random.default_rng(sum(numel) + 31 * n_d)
    case.init_state_gpu()
    case.init_state_oracle()
    for t in (1, 2, 3):
        ranges = _random_ranges(case.L.n_buckets, rng)
        say(f"  buckets numel={numel} cap={cap} n_d={n_d} r={rank} {gl} {om} t={t}: {ranges}")
        grads = case.grads_gpu(t)
        for b0, b1 in ranges:
            _step_buckets(case, t, grads, b0, b1)
        case.step_oracle(t, case.grads_oracle(t))
    torch.cuda.synchronize()
    case.compare("bucket ranges")
    for a, b in ((case.master, case.o_master), (case.m, case.o_m), (case.v, case.o_v)):
        assert_bitwise(a.cpu().numpy(), b, "state")
    pos = case.flat_pos if om == "ag_slot" else np.arange(case.S)
    assert_bitwise(u16(case.pout)[pos], case.o_p, "param")
    case.check_canaries(n_probe=4096)


def test_single_buckets_on_two_streams_equal_the_oracle():
    """ZeRO-2 call pattern: every bucket stepped on its own, the calls
    alternating between two streams (buckets are disjoint, so they may run
    concurrently), three steps: the oracle's whole-shard step bit for bit.
    The buckets are large enough for the small-region grid (one chunk per
    wave, several blocks per CU)."""
    case = _edge_case([10_000_003, 5_555_555, 77], 8_000_000, 8, 5, "compact", "ag_slot")
    case.init_state_gpu()
    case.init_state_oracle()
    main = torch.cuda.current_stream()
    side = [torch.cuda.Stream(), torch.cuda.Stream()]
    gl, om = z.GRAD_COMPACT, z.OUT_AG_SLOT
    for t in (1, 2, 3):
        grads = case.grads_gpu(t)
        for x in side:
            x.wait_stream(main)
        for b in range(case.L.n_buckets):
            z.zero_shard_step_buckets(case.L, case.hp_z, t, b, b + 1, grads, gl, case.master,
                                      case.m, case.v, case.pout, om, case.gout,
                                      stream=side[b % 2])
        for x in side:
            main.wait_stream(x)
        case.step_oracle(t, case.grads_oracle(t))
    torch.cuda.synchronize()
    case.compare("single buckets on two streams")
    case.check_canaries(n_probe=4096)


def _range_mask(case, b0, b1):
    """Shard indices of buckets [b0, b1)."""
    inside = np.zeros(case.S, bool)
    for b in range(b0, b1):
        lo = int(case.pl.shard_off[b])
        inside[lo:lo + int(case.pl.padded_len[b]) // case.w.n_d] = True
    return inside


@pytest.mark.parametrize("numel,cap,n_d,rank,gl,om,b0,b1", [
    ([70000, 3], 16384, 8, 7, "flat", "ag_slot", 1, 3),
    ([70000, 3], 16384, 8, 7, "flat", "ag_slot", 4, 5),     # the last bucket alone
    ([70000, 3], 16384, 8, 7, "flat", "ag_slot", 2, 5),
    ([1000, 37, 4096, 3], 1500, 4, 3, "compact", "shard", 0, 2),
    ([8192 * 6], 8192, 8, 2, "flat", "ag_slot", 3, 4),
    ([50000], 8008, 8, 3, "compact", "ag_slot", 5, 7),
])
def test_bucket_range_touches_only_its_slices(numel, cap, n_d, rank, gl, om, b0, b1):
    case = _edge_case(numel, cap, n_d, rank, gl, om)
    say(f"  bucket range [{b0}, {b1}) numel={numel} cap={cap} n_d={n_d} {gl} {om}")
    case.init_state_gpu()
    case.init_state_oracle()
    before = [case.master.cpu().numpy(), case.m.cpu().numpy(), case.v.cpu().numpy()]
    pout0 = u16(case.pout)
    gout0 = case.gout.cpu().numpy()
    _step_buckets(case, 1, case.grads_gpu(1), b0, b1)
    case.step_oracle(1, case.grads_oracle(1))
    torch.cuda.synchronize()
    inside = _range_mask(case, b0, b1)
    assert inside.any()
    for buf, old, exp in zip((case.master, case.m, case.v), before,
                             (case.o_master, case.o_m, case.o_v)):
        got = buf.cpu().numpy()
        assert_bitwise(got[inside], exp[inside], "state inside the range")
        assert_bitwise(got[~inside], old[~inside], "state outside the range")
    g = case.gout.cpu().numpy()
    assert_bitwise(g[inside], case.o_g[inside], "reduced gradient inside the range")
    assert_bitwise(g[~inside], gout0[~inside], "reduced gradient outside the range")
    p = u16(case.pout)
    pos = case.flat_pos if om == "ag_slot" else np.arange(case.S)
    assert_bitwise(p[pos[inside]], case.o_p[inside], "param inside the range")
    untouched = np.ones(p.size, bool)
    untouched[pos[inside]] = False
    assert_bitwise(p[untouched], pout0[untouched], "param outside the range")


@pytest.mark.parametrize("gl,om", [("flat", "ag_slot"), ("compact", "shard")])
def test_dim0_bucket_ranges_equal_the_whole_step(gl, om):
    """Per-parameter layout: tensors stepped in random groups equal one
    whole-shard step bit for bit (table launches over a tensor range; one
    plain shard range without flat addressing)."""
    shapes = [((k * 7) % 41 + 1, (k * 5) % 13 + 1) if k % 9 else (64, 64) for k in range(75)]
    numel = [int(np.prod(s)) for s in shapes]
    outs = []
    for split in (False, True):
        w = workloads.Workload("gpt2s_fsdp2", numel, 0, 4, 2, gl, om, 1, 1,
                               ("normal", 1e-3), ("normal", 0.02), ("normal", 1e-4),
                               ("absnormal", 1e-6), rows=[s[0] for s in shapes])
        case = Case(w)
        case.init_state_gpu()
        grads = case.grads_gpu(2)
        if split:
            for b0, b1 in _random_ranges(case.L.n_buckets, np.random.default_rng(5)):
                _step_buckets(case, 2, grads, b0, b1)
        else:
            case.step_gpu(2, grads)
        torch.cuda.synchronize()
        outs.append([case.master.cpu().numpy(), case.m.cpu().numpy(), case.v.cpu().numpy(),
                     u16(case.pout), case.gout.cpu().numpy()])
    for a, b in zip(*outs):
        assert_bitwise(a, b, "dim0 bucket ranges")


# ------------------------------------------------------------------ fp32 contributions
F32_EDGE = [
    ([1000, 37, 4096, 3], 1500, 4, 3, "flat", "ag_slot"),
    ([17], 0, 1, 0, "compact", "shard"),
    ([5, 0, 123, 64], 40, 3, 2, "flat", "ag_slot"),
    ([70000, 3], 16384, 8, 7, "flat", "ag_slot"),
    ([50000], 8008, 8, 3, "compact", "ag_slot"),
    ([20000, 20001], 0, 16, 15, "compact", "shard"),
    ([64 * 300 + 1], 6400, 64, 63, "compact", "shard"),
    ([100 * 97], 0, 100, 99, "flat", "ag_slot"),
    ([2 * 70000 + 1], 0, 2, 1, "flat", "ag_slot"),
    ([32 * 1040 * 3 + 45], 32 * 1040, 32, 31, "flat", "ag_slot"),
]


def _f32_contribs(case, t, flat):
    """fp32 contributions keyed like the bf16 ones; FLAT ones laid out over
    the padded flat buffer of each rank."""
    w = case.w
    pl = case.pl
    if flat:
        segs = [(int(po), int(so), int(ln), int(pln - ln))
                for so, ln, po, pln in zip(pl.stream_off, pl.len, pl.padded_off, pl.padded_len)]
        n = case.P
    else:
        segs, n = case.segs, case.S
    dev, host = [], []
    for q in range(w.n_d):
        k = synth.key(w.name, "grad", q, 0, t)
        g = torch.empty(n, dtype=torch.float32, device=DEV)
        synth.fill_device(g, segs, k, *w.grad)
        dev.append(g)
        host.append(synth.values_at(case.stream_pos, k, *w.grad, synth.OUT_F32))
    return dev, host


@pytest.mark.parametrize("numel,cap,n_d,rank,gl,om", F32_EDGE)
def test_f32_contributions_full_compare(numel, cap, n_d, rank, gl, om):
    case = _edge_case(numel, cap, n_d, rank, gl, om)
    say(f"  f32 numel={numel} cap={cap} n_d={n_d} r={rank} {gl} {om}: S={case.S}")
    case.init_state_gpu()
    case.init_state_oracle()
    for t in (1, 2, 3):
        dev, host = _f32_contribs(case, t, gl == "flat")
        case.step_gpu(t, dev)
        p, g = oracle.shard_step_f32(host, case.o_master, case.o_m, case.o_v, case.hp_o, t,
                                     want_grad=True)
        case.o_p, case.o_g = p, g
    torch.cuda.synchronize()
    case.compare("f32")
    for a, b in ((case.master, case.o_master), (case.m, case.o_m), (case.v, case.o_v)):
        assert_bitwise(a.cpu().numpy(), b, "state")
    case.check_canaries(n_probe=4096)


@pytest.mark.parametrize("launch", [(3, 64, 0), (0, 0, 1), (5000, 256, 0)])
def test_f32_launch_shape_invariance(launch):
    outs = []
    for lc in (None, launch):
        case = _edge_case([200_003, 77], 65_536, 16, 9, "flat", "ag_slot")
        case.init_state_gpu()
        dev, _ = _f32_contribs(case, 4, True)
        case.step_gpu(4, dev, launch=lc)
        torch.cuda.synchronize()
        outs.append([case.master.cpu().numpy(), u16(case.pout), case.gout.cpu().numpy()])
    for a, b in zip(*outs):
        assert_bitwise(a, b, f"f32 launch {launch}")


def test_no_sync_fp32_accumulators_feed_the_step():
    """Each rank's 4 micro-batches accumulate into fp32 (scaled by 1/4); the
    fp32 accumulators go to the step unrounded (fp32 Reduce-Scatter)."""
    w = workloads.Workload("flat1m", [3_000_001], 0, 8, 5, "compact", "ag_slot", 101, 1,
                           ("zero", 0.0), ("normal", 0.02), ("normal", 1e-4),
                           ("absnormal", 1e-6), n_micro=4, micro_grad=("normal", 2e-3))
    case = Case(w)
    case.init_state_gpu()
    case.init_state_oracle()
    accs, o_accs = [], []
    for q in range(w.n_d):
        acc = torch.empty(case.S, dtype=torch.float32, device=DEV)
        o_acc = np.zeros(case.S, np.float32)
        micro = torch.empty(case.S, dtype=torch.int16, device=DEV)
        for k in range(w.n_micro):
            key = synth.key(w.name, "micro_grad", q, k, w.t_first)
            synth.fill_device(micro, case.segs, key, *w.micro_grad)
            z.zero_grad_accumulate(acc, micro, 0.25, z.ACC_OVERWRITE if k == 0 else 0)
            oracle.accumulate(o_acc, synth.values_at(case.stream_pos, key, *w.micro_grad,
                                                      synth.OUT_BF16), 0.25, overwrite=(k == 0))
        accs.append(acc)
        o_accs.append(o_acc)
    case.step_gpu(w.t_first, accs)
    p, g = oracle.shard_step_f32(o_accs, case.o_master, case.o_m, case.o_v, case.hp_o, w.t_first,
                                 want_grad=True)
    case.o_p, case.o_g = p, g
    torch.cuda.synchronize()
    for a, b in zip(accs, o_accs):
        assert_bitwise(a.cpu().numpy(), b, "fp32 accumulator")
    case.compare("fp32 no_sync")
    assert_bitwise(case.master.cpu().numpy(), case.o_master, "master")


# ------------------------------------------------------------------ last micro-batch folded in
def _contribs(case, t, flat, kind, micro, dist, out_type):
    """Per-rank buffers keyed by (kind, rank, micro, t), COMPACT (S values in
    shard order) or FLAT (the padded flat buffer, zero padding), with the
    oracle's values at this rank's shard positions."""
    w, pl = case.w, case.pl
    if flat:
        segs = [(int(po), int(so), int(ln), int(pln - ln))
                for so, ln, po, pln in zip(pl.stream_off, pl.len, pl.padded_off, pl.padded_len)]
        n = case.P
    else:
        segs, n = case.segs, case.S
    dtype = torch.float32 if out_type == synth.OUT_F32 else torch.int16
    dev, host = [], []
    for q in range(w.n_d):
        k = synth.key(w.name, kind, q, micro, t)
        g = torch.empty(n, dtype=dtype, device=DEV)
        synth.fill_device(g, segs, k, *dist)
        dev.append(g)
        host.append(synth.values_at(case.stream_pos, k, *dist, out_type))
    return dev, host


def _fused_oracle(case, t, o_acc, o_micro, scale, contrib):
    """The separate calls the fused step stands for: each rank's last
    accumulate (emit bf16 without storing, or store fp32), then the step."""
    outs = []
    for a, g in zip(o_acc, o_micro):
        a = a.copy()
        if contrib == z.DTYPE_BF16:
            outs.append(oracle.accumulate(a, g, scale, overwrite=False, store_acc=False,
                                          emit=True))
        else:
            oracle.accumulate(a, g, scale, overwrite=False)
            outs.append(a)
    step = oracle.shard_step if contrib == z.DTYPE_BF16 else oracle.shard_step_f32
    case.o_p, case.o_g = step(outs, case.o_master, case.o_m, case.o_v, case.hp_o, t,
                              want_grad=True)


FUSED_EDGE = [
    ([1000, 37, 4096, 3], 1500, 4, 3, "flat", "ag_slot"),
    ([17], 0, 1, 0, "compact", "shard"),
    ([5, 0, 123, 64], 40, 3, 2, "flat", "ag_slot"),
    ([70000, 3], 16384, 8, 7, "flat", "ag_slot"),
    ([50000], 8008, 8, 3, "compact", "ag_slot"),
    ([20000, 20001], 0, 16, 15, "compact", "shard"),
    ([64 * 300 + 1], 6400, 64, 63, "compact", "shard"),
    ([100 * 97], 0, 100, 99, "flat", "ag_slot"),
    ([128 * 40 + 3], 0, 128, 127, "compact", "ag_slot"),
    ([2 * 70000 + 1], 0, 2, 1, "flat", "ag_slot"),
    ([32 * 1040 * 3 + 45], 32 * 1040, 32, 31, "compact", "shard"),
]


@pytest.mark.parametrize("contrib", [z.DTYPE_BF16, z.DTYPE_F32], ids=["bf16", "f32"])
@pytest.mark.parametrize("numel,cap,n_d,rank,gl,om", FUSED_EDGE)
def test_fused_last_micro_batch_full_compare(numel, cap, n_d, rank, gl, om, contrib):
    """zero_shard_step_accumulate against the oracle's last accumulate call
    followed by its step, every element, three steps."""
    case = _edge_case(numel, cap, n_d, rank, gl, om)
    say(f"  fused numel={numel} cap={cap} n_d={n_d} r={rank} {gl} {om} dtype={contrib}: "
        f"S={case.S}")
    case.init_state_gpu()
    case.init_state_oracle()
    flat = gl == "flat"
    for t in (1, 2, 3):
        acc, o_acc = _contribs(case, t, flat, "grad", 0, ("normal", 1e-3), synth.OUT_F32)
        mic, o_mic = _contribs(case, t, flat, "micro_grad", 3, ("normal", 2e-3), synth.OUT_BF16)
        z.zero_shard_step_accumulate(
            case.L, case.hp_z, t, acc, mic, 0.25, contrib,
            z.GRAD_FLAT if flat else z.GRAD_COMPACT, case.master, case.m, case.v, case.pout,
            z.OUT_AG_SLOT if om == "ag_slot" else z.OUT_SHARD, case.gout)
        _fused_oracle(case, t, o_acc, o_mic, 0.25, contrib)
    torch.cuda.synchronize()
    case.compare("fused")
    for a, b in ((case.master, case.o_master), (case.m, case.o_m), (case.v, case.o_v)):
        assert_bitwise(a.cpu().numpy(), b, "state")
    pos = case.flat_pos if om == "ag_slot" else np.arange(case.S)
    assert_bitwise(u16(case.pout)[pos], case.o_p, "param")
    case.check_canaries(n_probe=4096)


@pytest.mark.parametrize("launch", [(3, 64, 0), (0, 0, 1), (5000, 256, 0)])
def test_fused_launch_shape_invariance(launch):
    outs = []
    for lc in (None, launch):
        case = _edge_case([200_003, 77], 65_536, 16, 9, "flat", "ag_slot")
        case.init_state_gpu()
        acc, _ = _contribs(case, 4, True, "grad", 0, ("normal", 1e-3), synth.OUT_F32)
        mic, _ = _contribs(case, 4, True, "micro_grad", 3, ("normal", 2e-3), synth.OUT_BF16)
        z.zero_shard_step_accumulate(case.L, case.hp_z, 4, acc, mic, 0.25, z.DTYPE_BF16,
                                     z.GRAD_FLAT, case.master, case.m, case.v, case.pout,
                                     z.OUT_AG_SLOT, case.gout, launch=lc)
        torch.cuda.synchronize()
        outs.append([case.master.cpu().numpy(), u16(case.pout), case.gout.cpu().numpy()])
    for a, b in zip(*outs):
        assert_bitwise(a, b, f"fused launch {launch}")


@pytest.mark.timeout(600)
def test_accum1p3b_fused_sampled():
    """1.3e9 flat parameters, N_d = 8: every rank accumulates micro-batches
    1-3 (no_sync, 1/4 each), then the step takes each rank's accumulator and
    micro-batch 4 directly.  Sampled against the oracle's four accumulate
    calls and step; at full size every output also equals the separate last
    accumulate call + step (the same library's other route)."""
    w = workloads.get("accum1p3b")
    case = Case(w, sample_idx=np.arange(1))
    case.__init__(w, sample_idx=sample_indices(case.S, case.pl))
    case.init_state_gpu()
    case.init_state_oracle()
    S = case.S
    accs, lasts, o_accs, o_lasts = [], [], [], []
    for q in range(w.n_d):
        say(f"  accumulate rank {q}")
        acc = torch.empty(S, dtype=torch.float32, device=DEV)
        micro = torch.empty(S, dtype=torch.int16, device=DEV)
        o_acc = np.zeros(case.idx.size, np.float32)
        for k in range(w.n_micro):
            key = synth.key(w.name, "micro_grad", q, k, w.t_first)
            synth.fill_device(micro, case.segs, key, *w.micro_grad)
            o_micro = synth.values_at(case.stream_pos, key, *w.micro_grad, synth.OUT_BF16)
            if k + 1 < w.n_micro:
                z.zero_grad_accumulate(acc, micro, 1.0 / w.n_micro,
                                       z.ACC_OVERWRITE if k == 0 else 0)
                oracle.accumulate(o_acc, o_micro, 1.0 / w.n_micro, overwrite=(k == 0))
        accs.append(acc)
        lasts.append(micro)
        o_accs.append(o_acc)
        o_lasts.append(o_micro)
    say("  fused step t=101")
    z.zero_shard_step_accumulate(case.L, case.hp_z, w.t_first, accs, lasts, 1.0 / w.n_micro,
                                 z.DTYPE_BF16, z.GRAD_COMPACT, case.master, case.m, case.v,
                                 case.pout, z.OUT_AG_SLOT, case.gout)
    _fused_oracle(case, w.t_first, o_accs, o_lasts, 1.0 / w.n_micro, z.DTYPE_BF16)
    torch.cuda.synchronize()
    stats = case.compare("accum1p3b fused")
    say(f"  accum1p3b fused: exact matches {stats} of {case.idx.size}")
    case.check_canaries()
    fused_out = [case.master.cpu(), case.pout.cpu(), case.gout.cpu()]
    # the separate route on the same inputs, from the same initial state
    case.init_state_gpu()
    contribs = []
    for q in range(w.n_d):
        c = torch.empty(S, dtype=torch.int16, device=DEV)
        z.zero_grad_accumulate(accs[q], lasts[q], 1.0 / w.n_micro,
                               z.ACC_EMIT_BF16 | z.ACC_NO_STORE, c)
        contribs.append(c)
    del accs, lasts
    case.step_gpu(w.t_first, contribs)
    torch.cuda.synchronize()
    for a, b, what in zip(fused_out, [case.master.cpu(), case.pout.cpu(), case.gout.cpu()],
                          ("master", "param", "reduced grad")):
        assert torch.equal(a, b), f"fused and separate routes differ: {what}"


# ------------------------------------------------------------------ gather / reshard
GATHER = [
    ([1000, 37, 4096, 3], 1500, 4),
    ([5, 0, 123, 64], 40, 3),
    ([50000], 8008, 8),           # slice 1001: scalar path
    ([70000, 3], 16384, 8),       # vector path, short last bucket
    ([64 * 300 + 1], 6400, 64),
    ([256 * 33 + 7], 0, 256),
    ([2 * 4096 * 3 + 999, 77], 5000, 2),
    ([32 * 1040 * 3 + 45], 32 * 1040, 32),
]


def _rank_shards_bf16(pl, n_d, seed):
    out_h = []
    for q in range(n_d):
        segs = synth.shard_segments(pl.stream_off, pl.len, pl.padded_len, pl.shard_off, n_d, q)
        out_h.append(synth.fill_host(pl.shard_len, synth.OUT_BF16, segs,
                                     synth.key("gpt2s", "master", q, 0, seed), "normal", 0.02))
    return out_h


@pytest.mark.parametrize("numel,cap,n_d", GATHER)
def test_gather_params_matches_oracle(numel, cap, n_d):
    pl = oracle.plan(numel, cap, n_d)
    sh_h = _rank_shards_bf16(pl, n_d, 1)
    sh = [torch.from_numpy(x.view(np.int16)).to(DEV) for x in sh_h]
    L = z.Layout(numel, cap, n_d, 0)
    out = torch.full((pl.padded_total,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_gather_params(L, sh, out)
    torch.cuda.synchronize()
    assert_bitwise(u16(out), oracle.gather(sh_h, pl), "gathered flat buffer")
    if pl.n_buckets >= 3:
        # a bucket sub-range touches only its own buckets
        out.fill_(CANARY)
        z.zero_gather_params(L, sh, out, 1, 2)
        torch.cuda.synchronize()
        got = u16(out)
        exp = oracle.gather(sh_h, pl)
        lo, hi = pl.padded_off[1], pl.padded_off[1] + pl.padded_len[1]
        assert_bitwise(got[lo:hi], exp[lo:hi], "bucket 1")
        assert (got[:lo].view(np.int16) == CANARY).all() and (got[hi:].view(np.int16) == CANARY).all()


def test_gather_params_gpt2s_full():
    w = workloads.get("gpt2s")
    pl = oracle.plan(w.numel, w.cap, w.n_d)
    sh_h = _rank_shards_bf16(pl, w.n_d, 2)
    sh = [torch.from_numpy(x.view(np.int16)).to(DEV) for x in sh_h]
    out = torch.empty(pl.padded_total, dtype=torch.int16, device=DEV)
    z.zero_gather_params(z.Layout(w.numel, w.cap, w.n_d, 0), sh, out)
    torch.cuda.synchronize()
    assert_bitwise(u16(out), oracle.gather(sh_h, pl), "gpt2s gather")


def test_gather_params_gpt2s_fsdp2_full_and_tensor_range():
    """Per-parameter layout (148 tensors, table launches of 48): the whole
    gather, and a tensor range that leaves every other slot untouched."""
    w = workloads.get("gpt2s_fsdp2")
    pl = oracle.plan(w.numel, 0, w.n_d, rows=w.rows)
    sh_h = _rank_shards_bf16(pl, w.n_d, 4)
    sh = [torch.from_numpy(x.view(np.int16)).to(DEV) for x in sh_h]
    L = z.Layout(w.numel, 0, w.n_d, 0, rows=w.rows)
    exp = oracle.gather(sh_h, pl)
    out = torch.full((pl.padded_total,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_gather_params(L, sh, out)
    out2 = torch.full((pl.padded_total,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_gather_params(L, sh, out2, 50, 120)
    torch.cuda.synchronize()
    assert_bitwise(u16(out), exp, "gpt2s_fsdp2 gather")
    lo, hi = int(pl.padded_off[50]), int(pl.padded_off[119] + pl.padded_len[119])
    got = u16(out2)
    assert_bitwise(got[lo:hi], exp[lo:hi], "tensor range 50..119")
    assert (got[:lo].view(np.int16) == CANARY).all() and (got[hi:].view(np.int16) == CANARY).all()


RESHARD = [
    # numel, (cap, n_d) source, (cap, n_d, rank) destination
    ([1000, 37, 4096, 3], (1500, 4), (0, 2, 1)),
    ([5, 0, 123, 64], (40, 3), (16, 5, 4)),
    ([64 * 300 + 1], (6400, 64), (6400, 8, 7)),
    ([20000, 20001], (0, 16), (5000, 3, 0)),
    ([8], (0, 8), (0, 1, 0)),
]


@pytest.mark.parametrize("numel,src,dst", RESHARD)
def test_reshard_matches_oracle(numel, src, dst):
    ps = oracle.plan(numel, *src)
    pd = oracle.plan(numel, dst[0], dst[1])
    Ls = z.Layout(numel, src[0], src[1], 0)
    Ld = z.Layout(numel, *dst)
    for dt, out_type, tdt in ((np.float32, synth.OUT_F32, torch.float32),
                              (np.uint16, synth.OUT_BF16, torch.int16)):
        src_h = []
        for q in range(src[1]):
            segs = synth.shard_segments(ps.stream_off, ps.len, ps.padded_len, ps.shard_off,
                                        src[1], q)
            src_h.append(synth.fill_host(ps.shard_len, out_type, segs,
                                         synth.key("flat1m", "exp_avg", q), "normal", 1e-4))
        srcs = [torch.from_numpy(x.view(np.int16) if dt == np.uint16 else x).to(DEV) for x in src_h]
        out = torch.full((pd.shard_len,), 7, dtype=tdt, device=DEV)
        z.zero_reshard(Ls, srcs, Ld, out)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        exp = oracle.reshard(src_h, ps, pd, dst[2])
        assert_bitwise(got.view(dt) if dt == np.uint16 else got, exp, f"reshard {dt.__name__}")


def test_reshard_gpt2s_state_8_to_4_ranks_round_trip():
    """The optimizer state of GPT-2 small saved from 8 ranks (25 MiB buckets)
    re-cut for 4 ranks (12.5e6-element buckets) and back: the round trip is
    the identity and every piece equals the oracle's."""
    w = workloads.get("gpt2s")
    ps = oracle.plan(w.numel, w.cap, 8)
    pd = oracle.plan(w.numel, 12_500_000, 4)
    Ls = [z.Layout(w.numel, w.cap, 8, r) for r in range(8)]
    Ld = [z.Layout(w.numel, 12_500_000, 4, r) for r in range(4)]
    src_h = []
    for q in range(8):
        segs = synth.shard_segments(ps.stream_off, ps.len, ps.padded_len, ps.shard_off, 8, q)
        src_h.append(synth.fill_host(ps.shard_len, synth.OUT_F32, segs,
                                     synth.key("gpt2s", "master"), "normal", 0.02))
    srcs = [torch.from_numpy(x).to(DEV) for x in src_h]
    mid = []
    for r in range(4):
        out = torch.empty(pd.shard_len, dtype=torch.float32, device=DEV)
        z.zero_reshard(Ls[0], srcs, Ld[r], out)
        mid.append(out)
    torch.cuda.synchronize()
    assert_bitwise(mid[3].cpu().numpy(), oracle.reshard(src_h, ps, pd, 3), "8->4 rank 3")
    for r in range(8):
        back = torch.empty(ps.shard_len, dtype=torch.float32, device=DEV)
        z.zero_reshard(Ld[0], mid, Ls[r], back)
        torch.cuda.synchronize()
        assert_bitwise(back.cpu().numpy(), src_h[r], f"round trip rank {r}")


@pytest.mark.timeout(600)
def test_llama8b_pack_gather_reshard_full_size():
    """Full-size pack, gather and re-cut on the Llama-3-8B list (8.03e9
    elements; each call is split over several launches), bucketed and
    per-parameter (dim-0) shards.  Values are keyed
    by stream position, so the expected value of every position is known:
    sampled positions are checked against the generator and the oracle's
    layout, and every position against the concatenated tensors."""
    w = workloads.get("llama8b")
    pl = oracle.plan(w.numel, w.cap, 8)
    L0 = z.Layout(w.numel, w.cap, 8, 0)
    P, psi = pl.padded_total, sum(w.numel)
    key = synth.key(w.name, "grad", 0, 0, 1)
    dist = w.grad
    rng = np.random.default_rng(5)
    fpos = np.unique(np.concatenate([rng.integers(0, P, 1 << 18), np.arange(64),
                                     np.arange(P - 64, P)]))
    b = np.searchsorted(pl.padded_off, fpos, side="right") - 1
    off = fpos - pl.padded_off[b]
    xs = np.where(off < pl.len[b], pl.stream_off[b] + off, -1)
    expect = synth.values_at(xs, key, *dist, synth.OUT_BF16)

    say("  pack 291 tensors -> 8.03e9-element flat buffer")
    tens = [torch.empty(n, dtype=torch.int16, device=DEV) for n in w.numel]
    for t, segs in zip(tens, synth.tensor_segments(w.numel)):
        synth.fill_device(t, segs, key, *dist)
    flat = torch.full((P,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_bucket_pack(L0, tens, flat)
    torch.cuda.synchronize()
    assert_bitwise(flat[torch.from_numpy(fpos).to(DEV)].cpu().numpy().view(np.uint16), expect,
                   "packed flat buffer")
    stream_all = torch.cat([t.view(-1) for t in tens])
    del tens
    torch.cuda.empty_cache()

    say("  gather 8 shards -> flat buffer")
    shards = []
    for q in range(8):
        sh = torch.empty(pl.shard_len, dtype=torch.int16, device=DEV)
        synth.fill_device(sh, synth.shard_segments(pl.stream_off, pl.len, pl.padded_len,
                                                   pl.shard_off, 8, q), key, *dist)
        shards.append(sh)
    out = torch.full((P,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_gather_params(L0, shards, out)
    torch.cuda.synchronize()
    assert_bitwise(out[torch.from_numpy(fpos).to(DEV)].cpu().numpy().view(np.uint16), expect,
                   "gathered flat buffer")
    assert torch.equal(out, flat), "gather and pack disagree"
    del out, flat
    torch.cuda.empty_cache()

    say("  re-cut the 8 bf16 shards for one rank (the whole stream in order)")
    L1 = z.Layout(w.numel, w.cap, 1, 0)
    assert L1.shard == psi
    dst = torch.full((psi,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_reshard(L0, shards, L1, dst)
    torch.cuda.synchronize()
    xs1 = np.unique(rng.integers(0, psi, 1 << 18))
    assert_bitwise(dst[torch.from_numpy(xs1).to(DEV)].cpu().numpy().view(np.uint16),
                   synth.values_at(xs1, key, *dist, synth.OUT_BF16), "re-cut shard")
    assert torch.equal(dst, stream_all), "re-cut shard differs from the tensors in stream order"
    del shards
    torch.cuda.empty_cache()

    say("  per-parameter (dim-0) shards: gather, and re-cut for one bucketed rank")
    rows = [sh[1][0] for sh in w.shapes]
    pd = oracle.plan(w.numel, 0, 8, rows=rows)
    Ld = z.Layout(w.numel, 0, 8, 0, rows=rows)
    dshards = []
    for q in range(8):
        sh = torch.empty(pd.shard_len, dtype=torch.int16, device=DEV)
        synth.fill_device(sh, synth.shard_segments(pd.stream_off, pd.len, pd.padded_len,
                                                   pd.shard_off, 8, q), key, *dist)
        dshards.append(sh)
    dst.fill_(CANARY)
    z.zero_reshard(Ld, dshards, L1, dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, stream_all), "dim-0 re-cut differs from the tensors in stream order"
    dfull = torch.full((pd.padded_total,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_gather_params(Ld, dshards, dfull)
    torch.cuda.synchronize()
    dpos = np.unique(rng.integers(0, pd.padded_total, 1 << 18))
    db = np.searchsorted(pd.padded_off, dpos, side="right") - 1
    doff = dpos - pd.padded_off[db]
    dxs = np.where(doff < pd.len[db], pd.stream_off[db] + doff, -1)
    assert_bitwise(dfull[torch.from_numpy(dpos).to(DEV)].cpu().numpy().view(np.uint16),
                   synth.values_at(dxs, key, *dist, synth.OUT_BF16), "dim-0 gathered buffer")


# ------------------------------------------------------------------ FSDP2 per-parameter layout
def test_gpt2s_fsdp2_steps_full():
    """GPT-2-small list sharded per parameter along dim 0 over 8 ranks (the
    50257-row embedding leaves 7 padding rows on rank 7), FLAT contributions
    via pack, All-Gather slot output, 3 steps, every element compared."""
    case = Case(workloads.get("gpt2s_fsdp2"))
    stats = run_steps(case, full_check_steps=(1,))
    assert stats["master"] == case.S


DIM0_EDGE = [
    # shapes, n_d, rank, grad_layout, out_mode
    ([(4, 2), (4, 2), (4, 2)], 2, 1, "flat", "ag_slot"),
    ([(8, 4)], 4, 2, "compact", "shard"),
    ([(5, 3), (7,), (1, 9), (16, 16)], 4, 3, "flat", "ag_slot"),
    ([(5, 3), (7,), (1, 9), (16, 16)], 4, 0, "compact", "ag_slot"),
    ([(100, 24), (3, 8), (64, 64)], 8, 7, "flat", "shard"),
    ([(129, 64), (1000,)], 64, 63, "compact", "shard"),
    ([(129, 64), (1000,), (2, 3)], 64, 5, "flat", "ag_slot"),
    ([(64 * 40, 48), (1000,)], 64, 63, "compact", "shard"),   # 1024-element chunks + tail
    ([(33, 17), (1,), (250, 40)], 3, 2, "flat", "ag_slot"),
    # 75 tensors: three table launches mixing aligned and unaligned slices
    ([((k * 7) % 41 + 1, (k * 5) % 13 + 1) if k % 9 else (64, 64) for k in range(75)],
     4, 3, "flat", "ag_slot"),
    ([((k * 7) % 41 + 1, (k * 5) % 13 + 1) if k % 9 else (64, 64) for k in range(75)],
     8, 0, "compact", "ag_slot"),
    # runtime rank count: a table launch holds 92 slices
    ([((k * 7) % 41 + 1, (k * 5) % 13 + 1) if k % 9 else (64, 64) for k in range(75)],
     3, 2, "flat", "ag_slot"),
    ([((k * 7) % 41 + 1, (k * 5) % 13 + 1) if k % 9 else (64, 64) for k in range(230)],
     3, 1, "flat", "ag_slot"),
    # 400 tensors, 8 of them empty, many with only padding rows on rank 7:
    # three table launches of up to 191 slices
    ([(0, 5) if k % 50 == 3 else ((k * 11) % 37 + 1, (k * 3) % 7 + 1) if k % 5 else (2, 24)
      for k in range(400)], 8, 7, "flat", "ag_slot"),
    ([(0, 5) if k % 50 == 3 else ((k * 11) % 37 + 1, (k * 3) % 7 + 1) if k % 5 else (2, 24)
      for k in range(400)], 4, 1, "compact", "ag_slot"),
]


@pytest.mark.parametrize("shapes,n_d,rank,gl,om", DIM0_EDGE)
def test_dim0_layout_steps_full_compare(shapes, n_d, rank, gl, om):
    numel = [int(np.prod(s)) for s in shapes]
    w = workloads.Workload("gpt2s_fsdp2", numel, 0, n_d, rank, gl, om, 1, 1, ("normal", 1e-3),
                           ("normal", 0.02), ("normal", 1e-4), ("absnormal", 1e-6),
                           rows=[s[0] for s in shapes])
    case = Case(w)
    say(f"  dim0 shapes={shapes} n_d={n_d} r={rank} {gl} {om}: S={case.S}")
    case.init_state_gpu()
    case.init_state_oracle()
    for t in (1, 2):
        case.step_gpu(t, case.grads_gpu(t))
        case.step_oracle(t, case.grads_oracle(t))
    torch.cuda.synchronize()
    case.compare("dim0")
    for a, b in ((case.master, case.o_master), (case.m, case.o_m), (case.v, case.o_v)):
        assert_bitwise(a.cpu().numpy(), b, "state")
    pos = case.flat_pos if om == "ag_slot" else np.arange(case.S)
    assert_bitwise(u16(case.pout)[pos], case.o_p, "param")
    case.check_canaries(n_probe=4096)


@pytest.mark.parametrize("launch", [(3, 64, 0), (0, 0, 1), (5000, 128, 0)])
def test_dim0_launch_shape_invariance(launch):
    shapes = [((k * 7) % 41 + 1, (k * 5) % 13 + 1) if k % 9 else (64, 64) for k in range(75)]
    numel = [int(np.prod(s)) for s in shapes]
    outs = []
    for lc in (None, launch):
        w = workloads.Workload("gpt2s_fsdp2", numel, 0, 4, 2, "flat", "ag_slot", 1, 1,
                               ("normal", 1e-3), ("normal", 0.02), ("normal", 1e-4),
                               ("absnormal", 1e-6), rows=[s[0] for s in shapes])
        case = Case(w)
        case.init_state_gpu()
        case.step_gpu(2, case.grads_gpu(2), launch=lc)
        torch.cuda.synchronize()
        outs.append([case.master.cpu().numpy(), u16(case.pout), case.gout.cpu().numpy()])
    for a, b in zip(*outs):
        assert_bitwise(a, b, f"dim0 launch {launch}")


DIM0_DTYPE_CASES = [
    # shapes, n_d, rank, grad_layout, out_mode
    ([(5, 3), (7,), (1, 9), (16, 16), (33, 17), (300, 40)], 4, 3, "flat", "ag_slot"),
    ([(129, 64), (1000,), (2, 3), (64 * 40, 48)], 64, 5, "flat", "ag_slot"),
    ([(100, 24), (3, 8), (64, 64), (1000, 24)], 8, 7, "compact", "ag_slot"),
]


@pytest.mark.parametrize("contrib", ["f32", "fused_bf16", "fused_f32"])
@pytest.mark.parametrize("shapes,n_d,rank,gl,om", DIM0_DTYPE_CASES)
def test_dim0_f32_and_fused_steps_full_compare(shapes, n_d, rank, gl, om, contrib):
    """Per-parameter layouts with slot output run as table launches; fp32
    contributions and the fused last micro-batch (bf16 or fp32) through them,
    every element against the oracle, three steps.  Slices that end inside
    a chunk take the table kernel's element-wise path."""
    numel = [int(np.prod(sh)) for sh in shapes]
    case = _edge_case(numel, 0, n_d, rank, gl, om, rows=[sh[0] for sh in shapes])
    say(f"  dim0 {contrib} shapes={shapes} n_d={n_d} r={rank} {gl} {om}: S={case.S}")
    case.init_state_gpu()
    case.init_state_oracle()
    flat = gl == "flat"
    for t in (1, 2, 3):
        if contrib == "f32":
            dev, host = _f32_contribs(case, t, flat)
            case.step_gpu(t, dev)
            case.o_p, case.o_g = oracle.shard_step_f32(host, case.o_master, case.o_m, case.o_v,
                                                       case.hp_o, t, want_grad=True)
        else:
            dt = z.DTYPE_BF16 if contrib == "fused_bf16" else z.DTYPE_F32
            acc, o_acc = _contribs(case, t, flat, "grad", 0, ("normal", 1e-3), synth.OUT_F32)
            mic, o_mic = _contribs(case, t, flat, "micro_grad", 3, ("normal", 2e-3),
                                   synth.OUT_BF16)
            z.zero_shard_step_accumulate(
                case.L, case.hp_z, t, acc, mic, 0.25, dt,
                z.GRAD_FLAT if flat else z.GRAD_COMPACT, case.master, case.m, case.v,
                case.pout, z.OUT_AG_SLOT if om == "ag_slot" else z.OUT_SHARD, case.gout)
            _fused_oracle(case, t, o_acc, o_mic, 0.25, dt)
    torch.cuda.synchronize()
    case.compare(f"dim0 {contrib}")
    for a, b in ((case.master, case.o_master), (case.m, case.o_m), (case.v, case.o_v)):
        assert_bitwise(a.cpu().numpy(), b, "state")
    pos = case.flat_pos if om == "ag_slot" else np.arange(case.S)
    assert_bitwise(u16(case.pout)[pos], case.o_p, "param")
    case.check_canaries(n_probe=4096)


@pytest.mark.timeout(600)
def test_llama8b_fsdp2_sampled():
    w = workloads.get("llama8b_fsdp2")
    case = Case(w, sample_idx=np.arange(1))
    case.__init__(w, sample_idx=sample_indices(case.S, case.pl))
    run_steps(case)


@pytest.mark.parametrize("shapes,n_d", [([(5, 3), (7,), (1, 9), (16, 16)], 4),
                                        ([(129, 64), (1000,), (2, 3)], 64),
                                        ([(4, 2), (4, 2), (4, 2)], 2),
                                        ([((k * 7) % 41 + 1, (k * 5) % 13 + 1) if k % 9
                                          else (64, 64) for k in range(75)], 4)])
def test_dim0_gather_and_reshard(shapes, n_d):
    numel = [int(np.prod(s)) for s in shapes]
    rows = [s[0] for s in shapes]
    pd0 = oracle.plan(numel, 0, n_d, rows=rows)
    sh_h = _rank_shards_bf16(pd0, n_d, 3)
    sh = [torch.from_numpy(x.view(np.int16)).to(DEV) for x in sh_h]
    L0 = z.Layout(numel, 0, n_d, 0, rows=rows)
    out = torch.full((pd0.padded_total,), CANARY, dtype=torch.int16, device=DEV)
    z.zero_gather_params(L0, sh, out)
    torch.cuda.synchronize()
    assert_bitwise(u16(out), oracle.gather(sh_h, pd0), "dim0 gather")
    # re-cut dim0 -> bucketed -> dim0 (fp32), each piece against the oracle
    sh32_h = [synth.fill_host(pd0.shard_len, synth.OUT_F32,
                              synth.shard_segments(pd0.stream_off, pd0.len, pd0.padded_len,
                                                   pd0.shard_off, n_d, q),
                              synth.key("gpt2s", "exp_avg_sq"), "absnormal", 1e-6)
              for q in range(n_d)]
    sh32 = [torch.from_numpy(x).to(DEV) for x in sh32_h]
    pb = oracle.plan(numel, 7, 3)
    mid, mid_h = [], []
    for r in range(3):
        o = torch.full((pb.shard_len,), 5.0, dtype=torch.float32, device=DEV)
        z.zero_reshard(L0, sh32, z.Layout(numel, 7, 3, r), o)
        mid.append(o)
        mid_h.append(oracle.reshard(sh32_h, pd0, pb, r))
    torch.cuda.synchronize()
    for a, b in zip(mid, mid_h):
        assert_bitwise(a.cpu().numpy(), b, "dim0 -> bucketed")
    for r in range(n_d):
        o = torch.full((pd0.shard_len,), 5.0, dtype=torch.float32, device=DEV)
        z.zero_reshard(z.Layout(numel, 7, 3, 0), mid, z.Layout(numel, 0, n_d, r, rows=rows), o)
        torch.cuda.synchronize()
        assert_bitwise(o.cpu().numpy(), sh32_h[r], f"bucketed -> dim0 rank {r}")
    # dim0 -> dim0 with another rank count
    n2 = max(1, n_d // 2)
    pd2 = oracle.plan(numel, 0, n2, rows=rows)
    for r in range(n2):
        o = torch.full((pd2.shard_len,), 5.0, dtype=torch.float32, device=DEV)
        z.zero_reshard(L0, sh32, z.Layout(numel, 0, n2, r, rows=rows), o)
        torch.cuda.synchronize()
        assert_bitwise(o.cpu().numpy(), oracle.reshard(sh32_h, pd0, pd2, r), "dim0 -> dim0")


# ------------------------------------------------------------------ graph capture
def test_hip_graph_capture_of_accumulate_and_step():
    """The entry points launch kernels only (no allocation, memset or
    synchronisation), so a no_sync accumulation of 4 micro-batches for 2
    ranks followed by the shard step can be captured in one HIP graph.  Each
    of several replays (with eager work and synchronisations in between)
    equals the same sequence run eagerly, bit for bit."""
    numel, cap, n_d, rank, t = [700_001, 3_333], 65_536, 2, 1, 9
    L = z.Layout(numel, cap, n_d, rank)
    S, P = L.shard, L.padded
    hp = z.AdamW()
    rng = np.random.default_rng(31)

    def bf16(n, scale):
        return torch.from_numpy(oracle.round_bf16((rng.standard_normal(n) * scale)
                                                  .astype(np.float32)).view(np.int16)).to(DEV)

    micro = [[bf16(S, 2e-3) for _ in range(4)] for _ in range(n_d)]
    init = [torch.from_numpy((rng.standard_normal(S) * s).astype(np.float32)).to(DEV)
            for s in (0.02, 1e-4)] + [torch.from_numpy(
                np.abs(rng.standard_normal(S) * 1e-6).astype(np.float32)).to(DEV)]

    def make_bufs():
        return dict(acc=torch.zeros(S, dtype=torch.float32, device=DEV),
                    contrib=[torch.zeros(S, dtype=torch.int16, device=DEV) for _ in range(n_d)],
                    state=[x.clone() for x in init],
                    pout=torch.full((P,), CANARY, dtype=torch.int16, device=DEV))

    def sequence(b, stream=None):
        for q in range(n_d):
            for k in range(4):
                last = k == 3
                flags = (z.ACC_OVERWRITE if k == 0 else 0) | (
                    z.ACC_EMIT_BF16 | z.ACC_NO_STORE if last else 0)
                z.zero_grad_accumulate(b["acc"], micro[q][k], 0.25, flags,
                                       b["contrib"][q] if last else None, stream=stream)
        z.zero_shard_step(L, hp, t, b["contrib"], z.GRAD_COMPACT, *b["state"], b["pout"],
                          z.OUT_AG_SLOT, stream=stream)

    eager = make_bufs()
    expected = []
    for _ in range(3):
        sequence(eager)
        torch.cuda.synchronize()
        expected.append([x.cpu().numpy() for x in eager["state"]] + [u16(eager["pout"])])

    graphed = make_bufs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            sequence(graphed, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        junk = torch.ones(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        got = [x.cpu().numpy() for x in graphed["state"]] + [u16(graphed["pout"])]
        for a, b in zip(got, expected[r]):
            assert_bitwise(a, b, f"graph replay {r}")
        del junk


def test_hip_graph_capture_of_pack_fused_step_table_step_gather_and_reshard():
    """Every other entry point that launches kernels is capturable too: bucket
    pack (FLAT contributions), the step in two bucket ranges, the step with
    the last micro-batch folded in, a per-parameter (table) step, the
    parameter gather and a re-cut, captured in one HIP graph; each of several
    replays equals the same sequence run eagerly, bit for bit."""
    shapes = [((k * 7) % 41 + 1, (k * 5) % 13 + 1) if k % 9 else (64, 64) for k in range(40)]
    numel = [int(np.prod(s)) for s in shapes]
    rows = [s[0] for s in shapes]
    n_d, rank, t = 4, 1, 5
    Lb = z.Layout(numel, 1000, n_d, rank)                 # bucketed, FLAT contributions
    Ld = z.Layout(numel, 0, n_d, rank, rows=rows)         # per-parameter
    L2 = z.Layout(numel, 1000, 2, 0)                      # re-cut target
    hp = z.AdamW()
    rng = np.random.default_rng(77)

    def bf16(n, scale=1e-3):
        return torch.from_numpy(oracle.round_bf16((rng.standard_normal(n) * scale)
                                                  .astype(np.float32)).view(np.int16)).to(DEV)

    def f32(n, scale=1e-3):
        return torch.from_numpy((rng.standard_normal(n) * scale).astype(np.float32)).to(DEV)

    tens = [[bf16(n) for n in numel] for _ in range(n_d)]
    accs = [f32(Ld.shard) for _ in range(n_d)]
    micro = [bf16(Ld.shard, 2e-3) for _ in range(n_d)]
    shards = [bf16(Lb.shard, 0.02) for _ in range(n_d)]
    init = [f32(Lb.shard, 0.02), f32(Lb.shard, 1e-4), f32(Lb.shard, 1e-6).abs(),
            f32(Ld.shard, 0.02), f32(Ld.shard, 1e-4), f32(Ld.shard, 1e-6).abs()]

    def make_bufs():
        return dict(flat=[torch.zeros(Lb.padded, dtype=torch.int16, device=DEV)
                          for _ in range(n_d)],
                    state=[x.clone() for x in init],
                    pout_b=torch.full((Lb.padded,), CANARY, dtype=torch.int16, device=DEV),
                    pout_d=torch.full((Ld.padded,), CANARY, dtype=torch.int16, device=DEV),
                    full=torch.zeros(Lb.padded, dtype=torch.int16, device=DEV),
                    recut=torch.zeros(L2.shard, dtype=torch.float32, device=DEV))

    def sequence(b, stream=None):
        for q in range(n_d):
            z.zero_bucket_pack(Lb, tens[q], b["flat"][q], stream=stream)
        half = Lb.n_buckets // 2
        for b0, b1 in ((half, Lb.n_buckets), (0, half)):
            z.zero_shard_step_buckets(Lb, hp, t, b0, b1, b["flat"], z.GRAD_FLAT, *b["state"][:3],
                                      b["pout_b"], z.OUT_AG_SLOT, stream=stream)
        z.zero_shard_step_accumulate(Ld, hp, t, accs, micro, 0.25, z.DTYPE_BF16, z.GRAD_COMPACT,
                                     *b["state"][3:], b["pout_d"], z.OUT_AG_SLOT, stream=stream)
        z.zero_gather_params(Lb, shards, b["full"], stream=stream)
        z.zero_reshard(Lb, [b["state"][0]] * n_d, L2, b["recut"], stream=stream)

    def snapshot(b):
        return ([u16(x) for x in b["flat"]] + [x.cpu().numpy() for x in b["state"]] +
                [u16(b["pout_b"]), u16(b["pout_d"]), u16(b["full"]), b["recut"].cpu().numpy()])

    eager = make_bufs()
    expected = []
    for _ in range(3):
        sequence(eager)
        torch.cuda.synchronize()
        expected.append(snapshot(eager))

    graphed = make_bufs()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            sequence(graphed, stream=side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        junk = torch.ones(1 << 20, device=DEV).sum()
        torch.cuda.synchronize()
        for k, (a, b) in enumerate(zip(snapshot(graphed), expected[r])):
            assert_bitwise(a, b, f"graph replay {r}, buffer {k}")
        del junk
