"""Every element of the full-size shards against the CPU oracle.

The GPU runs the path at full size (inputs generated on the device by the
seeded generator); the shard is then streamed back in chunks, and for each
chunk the oracle steps the same inputs (the chunk's contributions and
pre-step state, copied back; a sample of them is first checked against the
generator's host implementation, so the oracle's inputs are pinned to the
host generator) and every output is compared: reduced gradient, master, m,
v and the bf16 parameters, bit for bit (NaN payloads aside), after the
stated bars (bitwise / 1e-6 relative / 1 ulp).

The knowledge card "FSDP" (kongchang.com), Core Facts, asks that the result
of a sharded update be checked as a whole, since accumulation order changes
with the parallel configuration; here the order is fixed and every element
of the shard is compared.
"""
import time

import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_step_amd as z
import oracle
import synth
from synth import workloads

from gpu_cases import (DEV, Case, assert_bf16_close, assert_bitwise, assert_f32_close,
                       assert_same_bits)

pytestmark = pytest.mark.gpu

CHUNK = 1 << 24
N_PIN = 2048          # inputs per chunk checked against the host generator


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _free_gpu_memory():
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _host(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


def _pin_inputs(case, c0, c1, arrays, keys_dists, out_type, rng):
    """A random sample of the chunk's copied-back inputs equals the host
    generator's values at the same parameters."""
    k = np.sort(rng.choice(c1 - c0, size=min(N_PIN, c1 - c0), replace=False))
    _, xs = case.pl.map(case.w.rank, c0 + k)
    for a, (key_, dist) in zip(arrays, keys_dists):
        exp = synth.values_at(xs, key_, *dist, out_type)
        assert_bitwise(a[k], exp, "device-filled input vs host generator")


def _compare_chunk(case, c0, c1, outs, o, what):
    gout, master, m, v, p = outs
    o_master, o_m, o_v, o_p, o_g = o
    assert_bitwise(gout, o_g, f"{what} reduced gradient")
    for got, exp, name in ((master, o_master, "master"), (m, o_m, "exp_avg"),
                           (v, o_v, "exp_avg_sq")):
        assert_f32_close(got, exp, f"{what} {name}")
        assert_same_bits(got, exp, f"{what} {name}")
    assert_bf16_close(p, o_p, f"{what} bf16 param")
    assert_same_bits(p, o_p, f"{what} bf16 param")


def _outputs(case, c0, c1):
    """The GPU's outputs for shard indices [c0, c1): reduced gradient,
    master, m, v, and the bf16 parameters (read from the All-Gather slots
    for slot output)."""
    sl = slice(c0, c1)
    if case.w.out_mode == "ag_slot":
        flat, _ = case.pl.map(case.w.rank, np.arange(c0, c1, dtype=np.int64))
        p = case.pout[torch.from_numpy(flat).to(DEV)].cpu().numpy().view(np.uint16)
    else:
        p = _host(case.pout[sl]).view(np.uint16)
    return (_host(case.gout[sl]), _host(case.master[sl]), _host(case.m[sl]), _host(case.v[sl]),
            p)


def run_whole_shard(name, f32=False):
    """One step of workload `name` on the GPU, then every element against the
    oracle; `f32`: binary32 contributions (the generator's values unrounded),
    stepped by zero_shard_step_ex with ZERO_DTYPE_F32."""
    w = workloads.get(name)
    assert w.grad_layout == "compact"
    case = Case(w, sample_idx=np.arange(1))
    S, t = case.S, w.t_first
    say(f"  {name}: S={S} N_d={w.n_d} t={t}" + (" fp32 contributions" if f32 else ""))
    case.init_state_gpu()
    if f32:
        grads = []
        for q in range(w.n_d):
            g = torch.empty(S, dtype=torch.float32, device=DEV)
            synth.fill_device(g, case.segs, synth.key(w.name, "grad", q, 0, t), *w.grad)
            grads.append(g)
    else:
        grads = case.grads_gpu(t)
    pre = [x.clone() for x in (case.master, case.m, case.v)]
    case.step_gpu(t, grads)
    torch.cuda.synchronize()
    say(f"  {name}: GPU step done; comparing in chunks of {CHUNK}")
    rng = np.random.default_rng(11)
    gkeys = [(synth.key(w.name, "grad", q, 0, t), w.grad) for q in range(w.n_d)]
    skeys = [(synth.key(w.name, k), d) for k, d in (("master", w.master),
                                                    ("exp_avg", w.exp_avg),
                                                    ("exp_avg_sq", w.exp_avg_sq))]
    t0 = time.time()
    for c0 in range(0, S, CHUNK):
        c1 = min(S, c0 + CHUNK)
        G = [_host(g[c0:c1]) if f32 else _host(g[c0:c1]).view(np.uint16) for g in grads]
        st = [_host(x[c0:c1]) for x in pre]
        _pin_inputs(case, c0, c1, G, gkeys, synth.OUT_F32 if f32 else synth.OUT_BF16, rng)
        _pin_inputs(case, c0, c1, st, skeys, synth.OUT_F32, rng)
        step = oracle.shard_step_f32 if f32 else oracle.shard_step
        o_p, o_g = step(G, *st, case.hp_o, t, want_grad=True, nthreads=synth.HOST_THREADS)
        _compare_chunk(case, c0, c1, _outputs(case, c0, c1), (*st, o_p, o_g),
                       f"{name} [{c0}, {c1})")
        if (c0 // CHUNK) % 16 == 0:
            say(f"  {name}: {c1} of {S} elements equal ({time.time() - t0:.0f} s)")
    return case


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["llama8b", "llama70b", "llama70b_t", "llama8b_fsdp2"])
def test_whole_shard_equals_oracle(name):
    """Llama-3-8B (N_d = 8, All-Gather slots, t = 1), Llama-70B and its
    padded-tail cut (N_d = 64, ZeRO-3 in place, t = 1001) and Llama-3-8B in
    the per-parameter dim-0 layout (in place): one step, every element."""
    case = run_whole_shard(name)
    if name == "llama70b_t":
        # padding positions stay +0 in every output
        pads = np.flatnonzero(case.pl.map(case.w.rank, np.arange(case.S - (1 << 22), case.S))[1]
                              < 0) + case.S - (1 << 22)
        assert pads.size > 0
        ix = torch.from_numpy(pads).to(DEV)
        for buf in (case.master, case.m, case.v, case.pout):
            assert not buf[ix].cpu().numpy().view(np.uint32 if buf.element_size() == 4
                                                   else np.uint16).any()
    if case.w.out_mode == "ag_slot":
        case.check_canaries()


@pytest.mark.timeout(900)
def test_whole_shard_with_fp32_contributions_equals_oracle():
    """The Llama-3-8B shard with binary32 contributions (a Reduce-Scatter in
    fp32, 58 bytes per element), one step, every element."""
    case = run_whole_shard("llama8b", f32=True)
    case.check_canaries()


@pytest.mark.timeout(900)
def test_accum1p3b_whole_shard_equals_oracle():
    """1.3e9 flat parameters, N_d = 8, rank 7: every rank accumulates its 4
    micro-batches scaled by 1/4 (no_sync; the last call emits the bf16
    contribution), then one step at t = 101.  Every contribution element and
    every output element is compared; the oracle forms the contributions
    itself from the micro-batch gradients."""
    w = workloads.get("accum1p3b")
    case = Case(w, sample_idx=np.arange(1))
    S, t, nd, nm = case.S, w.t_first, w.n_d, w.n_micro
    case.init_state_gpu()
    pre = [x.clone() for x in (case.master, case.m, case.v)]
    acc = torch.empty(S, dtype=torch.float32, device=DEV)
    micro = [[torch.empty(S, dtype=torch.int16, device=DEV) for _ in range(nm)]
             for _ in range(nd)]
    contribs = [torch.empty(S, dtype=torch.int16, device=DEV) for _ in range(nd)]
    mkeys = [[(synth.key(w.name, "micro_grad", q, k, t), w.micro_grad) for k in range(nm)]
             for q in range(nd)]
    for q in range(nd):
        for k in range(nm):
            synth.fill_device(micro[q][k], case.segs, mkeys[q][k][0], *w.micro_grad)
            last = k == nm - 1
            flags = (z.ACC_OVERWRITE if k == 0 else 0) | (
                z.ACC_EMIT_BF16 | z.ACC_NO_STORE if last else 0)
            z.zero_grad_accumulate(acc, micro[q][k], 1.0 / nm, flags,
                                   contribs[q] if last else None)
    case.step_gpu(t, contribs)
    torch.cuda.synchronize()
    say(f"  accum1p3b: GPU accumulate x{nd * nm} and step done; comparing")
    rng = np.random.default_rng(12)
    skeys = [(synth.key(w.name, k), d) for k, d in (("master", w.master),
                                                    ("exp_avg", w.exp_avg),
                                                    ("exp_avg_sq", w.exp_avg_sq))]
    for c0 in range(0, S, CHUNK):
        c1 = min(S, c0 + CHUNK)
        o_contribs = []
        for q in range(nd):
            mh = [_host(micro[q][k][c0:c1]).view(np.uint16) for k in range(nm)]
            _pin_inputs(case, c0, c1, mh, mkeys[q], synth.OUT_BF16, rng)
            o_acc = np.zeros(c1 - c0, np.float32)
            for k in range(nm):
                last = k == nm - 1
                out = oracle.accumulate(o_acc, mh[k], 1.0 / nm, overwrite=(k == 0),
                                        store_acc=not last, emit=last)
            assert_bitwise(_host(contribs[q][c0:c1]).view(np.uint16), out,
                           f"contribution of rank {q} [{c0}, {c1})")
            o_contribs.append(out)
        st = [_host(x[c0:c1]) for x in pre]
        _pin_inputs(case, c0, c1, st, skeys, synth.OUT_F32, rng)
        o_p, o_g = oracle.shard_step(o_contribs, *st, case.hp_o, t, want_grad=True,
                                     nthreads=synth.HOST_THREADS)
        _compare_chunk(case, c0, c1, _outputs(case, c0, c1), (*st, o_p, o_g),
                       f"accum1p3b [{c0}, {c1})")
    case.check_canaries()
