"""Helpers for the GPU parity tests: build seeded inputs on the GPU (synth),
run the path through the C ABI, and compute the expected values with the CPU
oracle on the same seeded inputs (all of them, or a sample of shard indices
that the oracle computes one by one).

Layout facts used to build inputs and expectations come from the oracle's
planner; the GPU path uses its own planner, so a disagreement shows up as a
parity failure.
"""
from __future__ import annotations

import numpy as np
import torch

import fsdp_sharded_optimizer_step_amd as z
import oracle
import synth
from synth import workloads

DEV = torch.device("cuda:0")
CANARY = -8531  # 0xDEAD as int16: fills the All-Gather buffer outside the slot


def u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def f32bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def assert_f32_close(got, exp, what, rel=1e-6):
    """Elementwise |got - exp| <= rel*|exp| (equal values, both zeros and
    same-payload NaNs pass)."""
    got = np.asarray(got, np.float32)
    exp = np.asarray(exp, np.float32)
    same = f32bits(got) == f32bits(exp)
    with np.errstate(invalid="ignore"):
        ok = same | (np.abs(got.astype(np.float64) - exp) <= rel * np.abs(exp.astype(np.float64)))
    ok |= np.isnan(got) & np.isnan(exp)
    if not ok.all():
        k = np.flatnonzero(~ok)
        raise AssertionError(f"{what}: {k.size} of {got.size} elements outside {rel} relative; "
                             f"first at {k[0]}: got {got[k[0]]!r} expected {exp[k[0]]!r}")
    return int(same.sum())


def assert_bf16_close(got, exp, what, ulps=1):
    got = np.asarray(got, np.uint16).astype(np.int32)
    exp = np.asarray(exp, np.uint16).astype(np.int32)
    same = got == exp
    same_sign = (got >> 15) == (exp >> 15)
    finite = ((got & 0x7F80) != 0x7F80) & ((exp & 0x7F80) != 0x7F80)
    near = same_sign & finite & (np.abs(got - exp) <= ulps)
    ok = same | near
    if not ok.all():
        k = np.flatnonzero(~ok)
        raise AssertionError(f"{what}: {k.size} of {got.size} bf16 values beyond {ulps} ulp; "
                             f"first at {k[0]}: got {got[k[0]]:#06x} expected {exp[k[0]]:#06x}")
    return int(same.sum())


def assert_same_bits(got, exp, what):
    """Bit-identical except where both values are NaN (IEEE arithmetic does
    not fix a NaN's payload).  got / exp: float32 arrays, or uint16 bf16
    patterns."""
    got = np.ascontiguousarray(got)
    exp = np.ascontiguousarray(exp)
    if got.dtype == np.float32:
        gb, eb = got.view(np.uint32), exp.astype(np.float32).view(np.uint32)
        both_nan = np.isnan(got) & np.isnan(exp)
    else:
        gb, eb = got.view(np.uint16), exp.view(np.uint16)
        both_nan = ((gb & 0x7F80) == 0x7F80) & ((gb & 0x7F) != 0) & \
                   ((eb & 0x7F80) == 0x7F80) & ((eb & 0x7F) != 0)
    bad = (gb != eb) & ~both_nan
    if bad.any():
        k = np.flatnonzero(bad)
        raise AssertionError(f"{what}: {k.size} of {got.size} values not bit-identical; first "
                             f"at {k[0]}: got {got[k[0]]!r} expected {exp[k[0]]!r}")


def assert_bitwise(got, exp, what):
    got = np.ascontiguousarray(got)
    exp = np.ascontiguousarray(exp)
    assert got.dtype.itemsize == exp.dtype.itemsize
    g = got.view(np.uint8).reshape(got.size, -1)
    e = exp.view(np.uint8).reshape(exp.size, -1)
    bad = (g != e).any(axis=1)
    if bad.any():
        k = np.flatnonzero(bad)
        raise AssertionError(f"{what}: {k.size} of {got.size} elements differ bitwise; "
                             f"first at {k[0]}: got {got[k[0]]!r} expected {exp[k[0]]!r}")


class Case:
    """One shard workload: layouts, GPU buffers and (sampled) oracle state."""

    def __init__(self, w: workloads.Workload, sample_idx=None):
        self.w = w
        self.pl = oracle.plan(w.numel, w.cap, w.n_d, rows=w.rows)
        self.L = z.Layout(w.numel, w.cap, w.n_d, w.rank, rows=w.rows)
        self.S, self.P = self.pl.shard_len, self.pl.padded_total
        self.hp_z = z.AdamW(**w.hp)
        self.hp_o = oracle.AdamW(**w.hp)
        self.segs = synth.shard_segments(self.pl.stream_off, self.pl.len, self.pl.padded_len,
                                         self.pl.shard_off, w.n_d, w.rank)
        # sample of shard indices checked by the oracle (None: all of them)
        self.idx = None if sample_idx is None else np.unique(np.asarray(sample_idx, np.int64))
        idx = np.arange(self.S) if self.idx is None else self.idx
        self.flat_pos, self.stream_pos = self.pl.map(w.rank, idx)

    # ---------------------------------------------------------------- state
    def init_state_gpu(self):
        w = self.w
        self.master = torch.empty(self.S, dtype=torch.float32, device=DEV)
        self.m = torch.empty_like(self.master)
        self.v = torch.empty_like(self.master)
        for buf, kind, dist in ((self.master, "master", w.master), (self.m, "exp_avg", w.exp_avg),
                                (self.v, "exp_avg_sq", w.exp_avg_sq)):
            synth.fill_device(buf, self.segs, synth.key(w.name, kind), dist[0], dist[1])
        n_out = self.P if w.out_mode == "ag_slot" else self.S
        self.pout = torch.full((n_out,), CANARY, dtype=torch.int16, device=DEV)
        self.gout = torch.empty(self.S, dtype=torch.float32, device=DEV)

    def init_state_oracle(self):
        w = self.w
        xs = self.stream_pos
        self.o_master = synth.values_at(xs, synth.key(w.name, "master"), *w.master, synth.OUT_F32)
        self.o_m = synth.values_at(xs, synth.key(w.name, "exp_avg"), *w.exp_avg, synth.OUT_F32)
        self.o_v = synth.values_at(xs, synth.key(w.name, "exp_avg_sq"), *w.exp_avg_sq,
                                   synth.OUT_F32)

    # ---------------------------------------------------------------- grads
    def grads_gpu(self, step: int):
        """The N_d contributions for this step, as the GPU path consumes them."""
        w = self.w
        if w.grad_layout == "compact":
            out = []
            for q in range(w.n_d):
                g = torch.empty(self.S, dtype=torch.int16, device=DEV)
                synth.fill_device(g, self.segs, synth.key(w.name, "grad", q, 0, step), *w.grad)
                out.append(g)
            return out
        # flat: per-tensor gradients packed into each rank's padded flat buffer
        tsegs = synth.tensor_segments(w.numel)
        tens = [torch.empty(max(1, n), dtype=torch.int16, device=DEV) for n in w.numel]
        flats = []
        for q in range(w.n_d):
            for t, n in enumerate(w.numel):
                if n:
                    synth.fill_device(tens[t], tsegs[t], synth.key(w.name, "grad", q, 0, step),
                                      *w.grad)
            flat = torch.full((self.P,), CANARY, dtype=torch.int16, device=DEV)
            z.zero_bucket_pack(self.L, tens, flat)
            flats.append(flat)
        return flats

    def grads_oracle(self, step: int):
        w = self.w
        return [synth.values_at(self.stream_pos, synth.key(w.name, "grad", q, 0, step), *w.grad,
                                synth.OUT_BF16) for q in range(w.n_d)]

    # ---------------------------------------------------------------- steps
    def step_gpu(self, t: int, grads, with_grad=True, launch=None):
        w = self.w
        gl = z.GRAD_FLAT if w.grad_layout == "flat" else z.GRAD_COMPACT
        om = z.OUT_AG_SLOT if w.out_mode == "ag_slot" else z.OUT_SHARD
        z.zero_shard_step(self.L, self.hp_z, t, grads, gl, self.master, self.m, self.v, self.pout,
                          om, self.gout if with_grad else None, launch=launch)

    def step_oracle(self, t: int, grads):
        p, g = oracle.shard_step(grads, self.o_master, self.o_m, self.o_v, self.hp_o, t,
                                 want_grad=True, nthreads=synth.HOST_THREADS)
        self.o_p, self.o_g = p, g

    # ---------------------------------------------------------------- compare
    def gather(self, t: torch.Tensor, idx):
        if idx is None:
            return t.cpu().numpy()
        return t[torch.from_numpy(idx).to(DEV)].cpu().numpy()

    def compare(self, what="", exact=True):
        """The stated bars (reduced gradient bitwise, fp32 state 1e-6
        relative, bf16 within 1 ulp), then, with `exact`, bit-identity of
        every output: the kernels run the oracle's operation sequence, so
        that is what holds.  Returns the exact-match counts."""
        idx = self.idx
        n_exact = {}
        assert_bitwise(self.gather(self.gout, idx), self.o_g, f"{what} reduced gradient")
        got = {"master": self.gather(self.master, idx), "exp_avg": self.gather(self.m, idx),
               "exp_avg_sq": self.gather(self.v, idx)}
        exp = {"master": self.o_master, "exp_avg": self.o_m, "exp_avg_sq": self.o_v}
        for k in got:
            n_exact[k] = assert_f32_close(got[k], exp[k], f"{what} {k}")
        pos = self.flat_pos if self.w.out_mode == "ag_slot" else (
            np.arange(self.S) if idx is None else idx)
        p = self.gather(self.pout, pos).view(np.uint16)
        n_exact["param"] = assert_bf16_close(p, self.o_p, f"{what} bf16 param")
        if exact:
            for k in got:
                assert_same_bits(got[k], exp[k], f"{what} {k}")
            assert_same_bits(p, self.o_p, f"{what} bf16 param")
        return n_exact

    def check_canaries(self, n_probe=1 << 20, seed=0):
        """All-Gather buffer positions outside this rank's slots are untouched."""
        if self.w.out_mode != "ag_slot":
            return
        rng = np.random.default_rng(seed)
        probe = np.unique(rng.integers(0, self.P, n_probe))
        mine = np.zeros(probe.size, bool)
        # a flat position f belongs to bucket b; it is ours iff its offset in
        # the bucket lies in [r*S_b, (r+1)*S_b)
        b = np.searchsorted(self.pl.padded_off, probe, side="right") - 1
        off = probe - self.pl.padded_off[b]
        sb = self.pl.padded_len[b] // self.w.n_d
        mine = (off >= self.w.rank * sb) & (off < (self.w.rank + 1) * sb)
        vals = self.gather(self.pout, probe[~mine])
        assert (vals == CANARY).all(), "All-Gather buffer written outside this rank's slot"


def sample_indices(S: int, pl, n_random=1 << 18, seed=0):
    """Random shard indices plus both ends and the first/last elements of
    several bucket slices (where addressing changes)."""
    rng = np.random.default_rng(seed)
    parts = [rng.integers(0, S, n_random), np.arange(min(S, 256)), np.arange(max(0, S - 256), S)]
    nb = pl.n_buckets
    for b in sorted(set([0, 1, nb // 2, nb - 2, nb - 1] + list(rng.integers(0, nb, 16)))):
        if 0 <= b < nb:
            lo = int(pl.shard_off[b])
            hi = lo + int(pl.padded_len[b]) // pl.n_d
            parts += [np.arange(lo, min(hi, lo + 16)), np.arange(max(lo, hi - 40), hi)]
    idx = np.unique(np.concatenate(parts))
    return idx[(idx >= 0) & (idx < S)]
