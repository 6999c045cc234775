"""One device allocation for a rank's step buffers, laid out by the
library's placement planner (zero_placement_plan in include/zero_shard.h).

torch provides the memory; this module only asks the planner for offsets
and carves typed views out of one uint8 pool.  No step of the update runs
here, and results do not depend on the placement.
"""
from __future__ import annotations

from .binding import (DTYPE_BF16, GRAD_FLAT, OUT_AG_SLOT, zero_placement_plan,
                      zero_shard_step, zero_shard_step_accumulate)

GiB = 1 << 30
LANE_BYTES = 32 * GiB   # MI355X, measured: lanes 32 GiB apart ...
N_LANES = 3             # ... three of them (a 96 GiB period)
ALIGN = 2 << 20
SLACK = 32 * GiB        # spare room measured to avoid the slow placements
# (spare bytes, shift step) tried in order by tuned_step_pool until a pool
# fits: the step's speed repeats with the arrangement's start with a period of
# about 96 GiB whose phase differs between devices, so the first search
# covers more than one period
SEARCH = ((128 * GiB, 8 * GiB), (64 * GiB, 8 * GiB), (SLACK, 4 * GiB))


class Pool:
    """specs: list of (name, numel, torch dtype, HBM bytes moved per shard
    element).  Allocates one pool on `device` and exposes `views[name]`.

    slack > 0 allocates that many extra bytes and lets `choose` pick where
    the planned arrangement starts: choose(views) -> milliseconds is called
    for the arrangement shifted by 0, shift_step, 2*shift_step, ... <= slack
    (views hold arbitrary bytes), and the fastest shift is kept.  HBM speed
    for the same arrangement depends on where the allocation lands
    physically, which user code cannot see, so it is measured."""

    def __init__(self, specs, device="cuda:0", lane_bytes=LANE_BYTES, n_lanes=N_LANES,
                 align=ALIGN, slack=0, choose=None, shift_step=4 * GiB):
        import torch
        self.specs = list(specs)
        self.sizes = [int(n) * torch.empty((), dtype=dt).element_size()
                      for _, n, dt, _ in self.specs]
        offs, need = zero_placement_plan(self.sizes, [tr for *_, tr in self.specs], lane_bytes,
                                         n_lanes, align)
        slack = max(0, int(slack)) // align * align
        self.plan = offs
        self.nbytes = need + slack
        self.buf = torch.zeros(max(self.nbytes, 1), dtype=torch.uint8, device=device)
        self.tuning = []
        shift = 0
        if choose is not None and slack > 0:
            step = max(align, int(shift_step) // align * align)
            for sh in range(0, slack + 1, step):
                self.tuning.append((sh, float(choose(self._carve(sh)))))
            shift = min(self.tuning, key=lambda x: x[1])[0]
        self.shift = shift
        self.views = self._carve(shift)
        self.offsets = {s[0]: o + shift for s, o in zip(self.specs, self.plan)}

    def _carve(self, shift):
        out = {}
        for (name, _, dt, _), o, b in zip(self.specs, self.plan, self.sizes):
            assert 0 <= o + shift and o + shift + b <= self.nbytes
            out[name] = self.buf[o + shift:o + shift + b].view(dt)
        return out

    def __getitem__(self, name):
        return self.views[name]

    @property
    def grads(self):
        """The contribution views g0, g1, ... in rank order."""
        out, q = [], 0
        while f"g{q}" in self.views:
            out.append(self.views[f"g{q}"])
            q += 1
        return out


def step_specs(layout, grad_dtype=None, grad_layout: int = 0, out_mode: int = OUT_AG_SLOT,
               reduced_grad: bool = False, accumulators: bool = False):
    """Buffer specs of one shard-step call on `layout`: contributions
    g0..g{N_d-1} (COMPACT: S elements, FLAT: P), with `accumulators` also the
    fp32 accumulators a0..a{N_d-1} of zero_shard_step_accumulate (the g's are
    then the bf16 last micro-batches), master / exp_avg / exp_avg_sq (S fp32),
    param_out (P bf16 slots or S in place) and optionally reduced_grad."""
    import torch
    gd = torch.int16 if grad_dtype is None else grad_dtype
    S, P = layout.shard, layout.padded
    ge = torch.empty((), dtype=gd).element_size()
    n_g = P if grad_layout == GRAD_FLAT else S
    specs = [(f"g{q}", n_g, gd, ge) for q in range(layout.n_d)]
    if accumulators:
        specs += [(f"a{q}", n_g, torch.float32, 4) for q in range(layout.n_d)]
    specs += [(k, S, torch.float32, 8) for k in ("master", "exp_avg", "exp_avg_sq")]
    specs += [("param_out", P if out_mode == OUT_AG_SLOT else S, torch.int16, 2)]
    if reduced_grad:
        specs += [("reduced_grad", S, torch.float32, 4)]
    return specs


def step_pool(layout, device="cuda:0", lane_bytes=LANE_BYTES, n_lanes=N_LANES, align=ALIGN,
              slack=0, choose=None, shift_step=4 * GiB, **spec_kw) -> Pool:
    """A Pool holding step_specs(layout, **spec_kw)."""
    return Pool(step_specs(layout, **spec_kw), device=device, lane_bytes=lane_bytes,
                n_lanes=n_lanes, align=align, slack=slack, choose=choose, shift_step=shift_step)


def step_timer(layout, hp, t: int, grad_layout: int, out_mode: int, reps: int = 4,
               accumulators: bool = False, reduced_grad: bool = False, micro_scale: float = 0.25,
               contrib_dtype: int = DTYPE_BF16, **_spec):
    """A `choose` callback: views -> milliseconds of the call the buffers are
    for (HIP events on the current stream, after one untimed call):
    zero_shard_step, or zero_shard_step_accumulate when the views hold the
    fp32 accumulators (spec flag `accumulators`); the reduced gradient is
    written when the views hold it (`reduced_grad`)."""
    import torch

    def ms(v):
        g = [v[f"g{q}"] for q in range(layout.n_d)]
        rg = v["reduced_grad"] if reduced_grad else None
        st = (v["master"], v["exp_avg"], v["exp_avg_sq"], v["param_out"])
        if accumulators:
            a = [v[f"a{q}"] for q in range(layout.n_d)]
            call = lambda: zero_shard_step_accumulate(layout, hp, t, a, g, micro_scale,
                                                      contrib_dtype, grad_layout, *st, out_mode,
                                                      rg)
        else:
            call = lambda: zero_shard_step(layout, hp, t, g, grad_layout, *st, out_mode, rg)
        call()
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            call()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    return ms


def tuned_step_pool(layout, hp, t: int, grad_layout: int = 0, out_mode: int = OUT_AG_SLOT,
                    slack=None, device="cuda:0", **spec_kw) -> Pool:
    """step_pool with spare bytes, its start chosen by timing the step at
    shifts over the spare room (the buffers' contents are arbitrary
    afterwards).  slack=None tries the (spare bytes, shift step) pairs of
    SEARCH in order until a pool fits on the device; an explicit `slack`
    (with `shift_step`, default 4 GiB) makes one attempt."""
    import torch
    choose = step_timer(layout, hp, t, grad_layout, out_mode,
                        accumulators=spec_kw.get("accumulators", False),
                        reduced_grad=spec_kw.get("reduced_grad", False))
    if slack is not None:
        return step_pool(layout, device=device, slack=slack, grad_layout=grad_layout,
                         out_mode=out_mode, choose=choose, **spec_kw)
    if "shift_step" in spec_kw:
        raise TypeError("tuned_step_pool: shift_step needs an explicit slack")
    last = None
    for sl, step in SEARCH:
        try:
            return step_pool(layout, device=device, slack=sl, grad_layout=grad_layout,
                             out_mode=out_mode, choose=choose, shift_step=step, **spec_kw)
        except torch.cuda.OutOfMemoryError as e:
            last = e
            torch.cuda.empty_cache()
    raise last
