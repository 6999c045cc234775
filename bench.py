"""Benchmark of the shard-local update on one MI355X.

A step is one call of zero_shard_step over one rank's whole shard: the
rank-ordered reduction of the N_d bf16 contributions, AdamW on the fp32
master / m / v shard, and the bf16 store into the rank's All-Gather slots (or
in place for ZeRO-3).  Inputs are seeded synthetic data generated on the GPU
before the timed region and stay resident in HBM; the optimizer state evolves
across the timed steps (t increases), the contributions are reused.

Default workload: the Llama-3-8B parameter list (8,030,261,248 parameters)
in 25 MiB buckets at N_d = 8, rank 7: a 1,003,782,656-element shard, eight
bf16 contributions (16 GB), 42 bytes per shard element.

Prints one JSON line (rank 0).  `value` is shard elements updated per second;
`roofline` is the step kernel's algorithmic HBM bytes per launch over its
average launch duration (HIP events on the launch stream); `cpu_baseline` is
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0
KERNEL_SOURCES = ["fsdp_sharded_optimizer_step_amd/csrc/shard_step.hip",
                  "fsdp_sharded_optimizer_step_amd/csrc/device_common.hpp"]

WORKLOAD_LABEL = {
    "llama8b": "Llama-3-8B shard: 8.03e9 params, 25 MiB buckets, N_d=8, rank 7, ZeRO-1/2 AG slot",
    "llama70b": "Llama-70B shard: 7.06e10 params, 25 MiB buckets, N_d=64, rank 63, ZeRO-3 in place",
    "llama70b_t": "Llama-70B shard: 12.5e6-element buckets (padded tails), N_d=64, rank 63, ZeRO-3",
}


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def step_kernel_name(n_d: int, mapped: bool) -> str:
    """The step_vec_kernel instantiation the library launches for bf16
    contributions (its name in rocprofv3 traces): <N_d or 0 for the runtime
    loop, flat addressing, ranks loaded per group, cache policy (7: every
    load and store non-temporal), dtype 0, pairs of 4-element pieces per
    lane (2 from N_d = 64 on, with 8 ranks per group)>."""
    nd = n_d if n_d in (2, 4, 8, 16, 32, 64) else 0
    pairs = 2 if nd >= 64 else 1
    gmax = 8 if pairs > 1 else 16
    group = min(gmax, nd - 1) if nd > 1 else 1
    b = lambda x: "true" if x else "false"
    return f"step_vec_kernel<{nd}, {b(mapped)}, {group}, 7, 0, {pairs}>"


def traffic_from_profiles(workload: str, n_launch_bytes: float):
    """Measured HBM bytes per launch from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(ROOT, "profiles", f"shard_step_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_hash") != kernel_hash():
        return None
    return d.get("hbm_bytes_per_launch")


class Inputs:
    """The buffers of one shard-step call: `grads` (N_d contributions),
    `accs` (N_d fp32 accumulators, or None), `state` [master, m, v], `pout`."""

    def __init__(self, views, n_d, pool=None):
        self.grads = [views[f"g{q}"] for q in range(n_d)]
        self.accs = [views[f"a{q}"] for q in range(n_d)] if "a0" in views else None
        self.state = [views["master"], views["exp_avg"], views["exp_avg_sq"]]
        self.pout = views["param_out"]
        self.pool = pool


TUNE_SLACK = 32 << 30   # extra pool bytes over which the tuned placement may shift
# the main workload's pool: the library helper's search, (spare bytes, shift
# step) pairs tried in order until a pool fits
from fsdp_sharded_optimizer_step_amd.placement import SEARCH as MAIN_TUNE  # noqa: E402


def step_call(z, L, hp, t, grad_layout, out_mode, fused=False):
    """views -> one step call on those buffers (for placement tuning)."""
    def call(v):
        nd = L.n_d
        g = [v[f"g{q}"] for q in range(nd)]
        st = (v["master"], v["exp_avg"], v["exp_avg_sq"], v["param_out"])
        if fused:
            z.zero_shard_step_accumulate(L, hp, t, [v[f"a{q}"] for q in range(nd)], g, 0.25,
                                         z.DTYPE_BF16, grad_layout, *st[:3], st[3], out_mode)
        else:
            z.zero_shard_step(L, hp, t, g, grad_layout, *st[:3], st[3], out_mode)
    return call


def mix_choose(L):
    """views -> milliseconds of the same-mix probe on the step's buffers: the
    placement search of the timed workloads, so that the step kernel's
    dispatches in a kernel trace are the warm-up and the timed calls only."""
    import measure

    def choose(v):
        g = [v[f"g{q}"] for q in range(L.n_d)]
        return measure.mix_ms(g, [v["master"], v["exp_avg"], v["exp_avg_sq"]], v["param_out"],
                              L.shard)
    return choose


def make_inputs(z, synth, w, L, placement="tuned", grad_dtype=None, accumulators=False,
                grad_micro=0, call=None, tune=((TUNE_SLACK, 4 << 30),), choose=None):
    """Buffers for workload w on layout L filled with the workload's seeded
    values (contributions keyed (grad, rank, grad_micro, t_first); FLAT ones
    over the padded flat buffer), the output zeroed.  placement "tuned": one
    pool laid out by zero_placement_plan with spare bytes, the arrangement's
    start chosen by timing `call` (views -> one call) at shifts over the
    spare room (`tune`: (spare bytes, shift step) pairs tried in order until
    a pool fits), or by `choose` (views -> milliseconds) when given;
    "planned": the same pool without spare bytes; "compact": three lanes
    just large enough for the buffers, no spare bytes; "separate": one torch
    allocation per buffer."""
    import torch
    from fsdp_sharded_optimizer_step_amd import placement as zp
    dev = torch.device("cuda:0")
    flat = w.grad_layout == "flat"
    gl = z.GRAD_FLAT if flat else z.GRAD_COMPACT
    om = z.OUT_AG_SLOT if w.out_mode == "ag_slot" else z.OUT_SHARD
    specs = zp.step_specs(L, grad_dtype=grad_dtype, grad_layout=gl, out_mode=om,
                          accumulators=accumulators)
    if placement not in ("tuned", "planned", "compact", "separate"):
        raise ValueError(placement)
    pool = None
    if placement == "compact":
        # three lanes just large enough for the buffers (a pool of about
        # 1.2x their size), at the allocation's own start: no spare room,
        # no timed search
        total = sum(n * torch.empty((), dtype=dt).element_size() for _, n, dt, _ in specs)
        lane = -(-total // (3 << 30)) << 30
        pool = zp.Pool(specs, device=dev, lane_bytes=lane)
        views = pool.views
    elif placement in ("tuned", "planned"):
        if placement != "tuned":
            choose = None
        elif choose is None:
            if call is None:
                call = step_call(z, L, z.AdamW(**w.hp), w.t_first, gl, om, fused=accumulators)
            timed = make_timer(torch.cuda.current_stream())
            choose = lambda v: timed(lambda: call(v), reps=4)
        tries = tune if placement == "tuned" else ((0, 4 << 30),)
        for slack, step in tries:
            try:
                pool = zp.Pool(specs, device=dev, slack=slack, choose=choose, shift_step=step)
                views = pool.views
                break
            except torch.cuda.OutOfMemoryError:
                torch.cuda.empty_cache()
                print(f"# {placement} pool with {slack >> 30} GiB spare does not fit",
                      file=sys.stderr, flush=True)
        if pool is None:
            # a device without room for the pool's spare lanes: one
            # allocation per buffer instead (reported as such)
            print(f"# {placement} pool does not fit; separate allocations", file=sys.stderr,
                  flush=True)
            placement = "separate"
    if placement == "separate":
        views = {name: torch.empty(n, dtype=dt, device=dev) for name, n, dt, _ in specs}
    so, ln, po, pln, sh = (list(x) for x in zip(*L.buckets()))
    segs = synth.shard_segments(so, ln, pln, sh, w.n_d, w.rank)
    gsegs = [(p0, s0, l, pl - l) for s0, l, p0, pl in zip(so, ln, po, pln)] if flat else segs
    gdist = w.micro_grad if w.n_micro else w.grad
    for q in range(w.n_d):
        synth.fill_device(views[f"g{q}"], gsegs,
                          synth.key(w.name, "grad", q, grad_micro, w.t_first), *gdist)
        if accumulators:
            synth.fill_device(views[f"a{q}"], gsegs, synth.key(w.name, "grad", q, 0, w.t_first),
                              *gdist)
    for kind, dist, name in (("master", w.master, "master"), ("exp_avg", w.exp_avg, "exp_avg"),
                             ("exp_avg_sq", w.exp_avg_sq, "exp_avg_sq")):
        synth.fill_device(views[name], segs, synth.key(w.name, kind), *dist)
    views["param_out"].zero_()
    torch.cuda.synchronize()
    return Inputs(views, w.n_d, pool), segs


def cpu_baseline(w, segs, S, target_s=12.0):
    """The CPU oracle on a contiguous sample of the shard (inputs generated
    outside the timed region), all host threads up to 16."""
    import numpy as np

    import oracle
    import synth
    threads = max(1, min(16, os.cpu_count() or 1))

    def sample_inputs(n):
        sub, left = [], n
        for d, x0, nr, npd in segs:
            if left <= 0:
                break
            take_r = min(nr, left)
            take_p = min(npd, left - take_r)
            sub.append((d if not sub else sum(s[2] + s[3] for s in sub), x0, take_r, take_p))
            left -= take_r + take_p
        n = sum(s[2] + s[3] for s in sub)
        G = [synth.fill_host(n, synth.OUT_BF16, sub,
                             synth.key(w.name, "grad", q, 0, w.t_first), *w.grad)
             for q in range(w.n_d)]
        st = [synth.fill_host(n, synth.OUT_F32, sub, synth.key(w.name, k), *dist)
              for k, dist in (("master", w.master), ("exp_avg", w.exp_avg),
                              ("exp_avg_sq", w.exp_avg_sq))]
        return n, G, st

    hp = oracle.AdamW(**w.hp)
    # the sample: 2^29 / N_d contiguous shard elements (64M at N_d = 8, 8M
    # at N_d = 64), stepped repeatedly (t advancing) until about target_s of
    # CPU work has been timed; the number of steps comes from one untimed
    # step of the same sample
    n = int(min(S, (1 << 29) // w.n_d))
    n, G, st = sample_inputs(n)
    t0 = time.perf_counter()
    oracle.shard_step(G, *st, hp, w.t_first, nthreads=threads)
    pilot = max(1e-6, time.perf_counter() - t0)
    reps = max(1, int(round(target_s / pilot)))
    t0 = time.perf_counter()
    for k in range(reps):
        oracle.shard_step(G, *st, hp, w.t_first + 1 + k, nthreads=threads)
    dt = time.perf_counter() - t0
    # one host thread on the first 2^22 elements of the same sample, about 3 s
    n1 = min(n, 1 << 22)
    G1, st1 = [g[:n1].copy() for g in G], [x[:n1].copy() for x in st]
    del G, st
    t0 = time.perf_counter()
    oracle.shard_step(G1, *st1, hp, w.t_first, nthreads=1)
    pilot1 = max(1e-6, time.perf_counter() - t0)
    reps1 = max(1, int(round(3.0 / pilot1)))
    t0 = time.perf_counter()
    for k in range(reps1):
        oracle.shard_step(G1, *st1, hp, w.t_first + 2 + k, nthreads=1)
    dt1 = time.perf_counter() - t0
    return {"value": n * reps / dt, "unit": "elem/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} elements of the same shard (inputs generated untimed), "
                      f"{reps} consecutive steps, {dt:.1f} s on {threads} host threads",
            "gbps": n * reps * (2 * w.n_d + 26) / dt / 1e9,
            "single_thread": {"value": n1 * reps1 / dt1, "unit": "elem/s", "cores": 1,
                              "sample": f"first {n1} elements, {reps1} steps, {dt1:.1f} s"}}


def make_timer(stream):
    """fn -> average milliseconds per call (HIP events on `stream`, one untimed call first)."""
    import torch

    def timed(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps
    return timed


def make_graph_timer(stream):
    """fn(stream) -> average milliseconds per replay of a HIP graph holding
    one fn call (captured on a side stream), so the host's marshalling of
    many pointers per call is not what is timed."""
    import torch
    timed = make_timer(stream)

    def gtimed(fn, reps=10):
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(g, stream=side):
                fn(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        ms = timed(g.replay, reps=reps)
        del g
        return ms
    return gtimed


def aux_kernels(z, synth, workloads, placement):
    """Pack (gpt2s list, one rank's 124M-element flat buffer), the gpt2s
    launch sequence (8 ranks pack, then the step), the no_sync
    accumulate sequence (accum1p3b shard: 4 calls for one rank) and the whole
    accum1p3b job (8 ranks accumulate, then the step; the last accumulate
    separate or folded into the step), timed with HIP events.  With a pool
    placement the buffers of each measurement share one tuned pool."""
    import torch
    from fsdp_sharded_optimizer_step_amd import placement as zp
    dev = torch.device("cuda:0")
    out = []
    timed = make_timer(torch.cuda.current_stream())

    def buffers(specs, call):
        """name -> view (pool) or tensor (separate); `call(views)` is timed to
        choose the pool's start."""
        if placement == "separate":
            return {n: torch.zeros(k, dtype=dt, device=dev) for n, k, dt, _ in specs}
        pool = zp.Pool(specs, device=dev, slack=TUNE_SLACK if placement == "tuned" else 0,
                       choose=(lambda v: timed(lambda: call(v), reps=3))
                       if placement == "tuned" else None)
        return pool.views

    def record(kernel, desc, nbytes, ms):
        out.append({"kernel": kernel, "workload": desc, "bytes_per_call": nbytes, "ms": ms,
                    "GBps": nbytes / (ms * 1e-3) / 1e9,
                    "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS})

    # bucket pack: every tensor is read while the flat buffer is written
    w = workloads.get("gpt2s")
    L = z.Layout(w.numel, w.cap, w.n_d, w.rank)
    specs = [(f"t{k}", n, torch.int16, float(n)) for k, n in enumerate(w.numel)]
    specs += [("flat", L.padded, torch.int16, float(L.padded))]
    nt = len(w.numel)
    gtimed = make_graph_timer(torch.cuda.current_stream())
    pack = lambda v, stream=None: z.zero_bucket_pack(L, [v[f"t{k}"] for k in range(nt)],
                                                     v["flat"], stream=stream)
    v = buffers(specs, pack)
    for k, segs in enumerate(synth.tensor_segments(w.numel)):
        synth.fill_device(v[f"t{k}"], segs, synth.key(w.name, "grad", 0, 0, 1), *w.grad)
    record("pack_kernel", "gpt2s: 148 tensors -> 124,439,808-element flat buffer, 25 MiB "
           "buckets (HIP graph replays; the same 249 MB of sources every replay)",
           2 * L.psi + 2 * L.padded, gtimed(lambda st: pack(v, st)))
    del v
    torch.cuda.empty_cache()
    # the 8 simulated ranks' packs, each from its own 148 tensors (2 GB of
    # sources in all, so none is still held by the 256 MB MALL when read)
    nd = w.n_d
    specs = [(f"t{q}_{k}", n, torch.int16, float(n)) for q in range(nd)
             for k, n in enumerate(w.numel)]
    specs += [(f"flat{q}", L.padded, torch.int16, float(L.padded)) for q in range(nd)]

    def packs(v, stream=None):
        for q in range(nd):
            z.zero_bucket_pack(L, [v[f"t{q}_{k}"] for k in range(nt)], v[f"flat{q}"],
                               stream=stream)

    v = buffers(specs, packs)
    for q in range(nd):
        for k, segs in enumerate(synth.tensor_segments(w.numel)):
            synth.fill_device(v[f"t{q}_{k}"], segs, synth.key(w.name, "grad", q, 0, 1), *w.grad)
    record("pack_kernel x8", f"gpt2s: {nd} ranks each pack their own 148 tensors into their "
           "own flat buffer (HIP graph replays)", nd * (2 * L.psi + 2 * L.padded),
           gtimed(lambda st: packs(v, st)))
    del v
    torch.cuda.empty_cache()

    # the gpt2s launch sequence of one optimizer step: every simulated rank
    # packs its own 148 tensors into its flat bucket buffer, then the step
    # reads rank r's slice of each bucket from the 8 buffers (FLAT) and
    # writes the All-Gather slots
    nd = w.n_d
    hp = z.AdamW(**w.hp)
    specs = [(f"t{q}_{k}", n, torch.int16, float(n)) for q in range(nd)
             for k, n in enumerate(w.numel)]
    specs += [(f"flat{q}", L.padded, torch.int16, float(L.padded)) for q in range(nd)]
    specs += [(k, L.shard, torch.float32, 8.0) for k in ("master", "exp_avg", "exp_avg_sq")]
    specs += [("param_out", L.padded, torch.int16, 2.0)]

    def gpt2s_job(v, stream=None):
        for q in range(nd):
            z.zero_bucket_pack(L, [v[f"t{q}_{k}"] for k in range(nt)], v[f"flat{q}"],
                               stream=stream)
        z.zero_shard_step(L, hp, w.t_first, [v[f"flat{q}"] for q in range(nd)], z.GRAD_FLAT,
                          v["master"], v["exp_avg"], v["exp_avg_sq"], v["param_out"],
                          z.OUT_AG_SLOT, stream=stream)

    v = buffers(specs, gpt2s_job)
    tsegs = synth.tensor_segments(w.numel)
    for q in range(nd):
        for k, segs in enumerate(tsegs):
            synth.fill_device(v[f"t{q}_{k}"], segs, synth.key(w.name, "grad", q, 0, 1), *w.grad)
    record("pack_kernel x8 + step_vec_kernel", f"gpt2s step: {nd} ranks pack 148 tensors each, "
           "then the shard step on rank 7's slices (FLAT, AG slot; HIP graph replays)",
           nd * (2 * L.psi + 2 * L.padded) + L.shard * (2 * nd + 26),
           gtimed(lambda st: gpt2s_job(v, st)))
    del v
    torch.cuda.empty_cache()

    # one rank's no_sync sequence on the accum1p3b shard
    w = workloads.get("accum1p3b")
    L = z.Layout(w.numel, w.cap, w.n_d, w.rank)
    S = L.shard
    so, ln, _, pln, sh = (list(x) for x in zip(*L.buckets()))
    segs = synth.shard_segments(so, ln, pln, sh, w.n_d, w.rank)
    scale = 1.0 / w.n_micro
    nm, nd = w.n_micro, w.n_d

    def seq(v):
        for k in range(nm):
            last = k == nm - 1
            flags = (z.ACC_OVERWRITE if k == 0 else 0) | (
                z.ACC_EMIT_BF16 | z.ACC_NO_STORE if last else 0)
            z.zero_grad_accumulate(v["acc"], v[f"m{k}"], scale, flags, v["emit"] if last else None)

    specs = [("acc", S, torch.float32, 8.0)] + [(f"m{k}", S, torch.int16, 2.0) for k in range(nm)]
    specs += [("emit", S, torch.int16, 2.0)]
    v = buffers(specs, seq)
    for k in range(nm):
        synth.fill_device(v[f"m{k}"], segs, synth.key(w.name, "micro_grad", 0, k, w.t_first),
                          *w.micro_grad)
    record("accum_vec_kernel", "accum1p3b: 162,500,000-element shard, 4 micro-batches "
           "(overwrite, add, add, add+emit bf16 without fp32 store)", S * (6 + 10 + 10 + 8),
           timed(lambda: seq(v), reps=5))
    del v
    torch.cuda.empty_cache()

    # the whole no_sync step of accum1p3b: every rank accumulates its 4
    # micro-batches, then the shard step -- the last accumulate as its own
    # call (emit bf16) or folded into the step (zero_shard_step_accumulate)
    hp = z.AdamW(**w.hp)

    def job(v, fused):
        for q in range(nd):
            for k in range(nm - (1 if fused else 0)):
                last = k == nm - 1
                flags = (z.ACC_OVERWRITE if k == 0 else 0) | (
                    z.ACC_EMIT_BF16 | z.ACC_NO_STORE if last else 0)
                z.zero_grad_accumulate(v[f"a{q}"], v[f"m{q}_{k}"], scale, flags,
                                       v[f"c{q}"] if last else None)
        st = (v["master"], v["exp_avg"], v["exp_avg_sq"], v["param_out"])
        if fused:
            z.zero_shard_step_accumulate(L, hp, w.t_first, [v[f"a{q}"] for q in range(nd)],
                                         [v[f"m{q}_{nm - 1}"] for q in range(nd)], scale,
                                         z.DTYPE_BF16, z.GRAD_COMPACT, *st, z.OUT_AG_SLOT)
        else:
            z.zero_shard_step(L, hp, w.t_first, [v[f"c{q}"] for q in range(nd)], z.GRAD_COMPACT,
                              *st, z.OUT_AG_SLOT)

    specs = [(f"a{q}", S, torch.float32, 8.0) for q in range(nd)]
    specs += [(f"m{q}_{k}", S, torch.int16, 2.0) for q in range(nd) for k in range(nm)]
    specs += [(f"c{q}", S, torch.int16, 2.0) for q in range(nd)]
    specs += [(k, S, torch.float32, 8.0) for k in ("master", "exp_avg", "exp_avg_sq")]
    specs += [("param_out", L.padded, torch.int16, 2.0)]
    v = buffers(specs, lambda v: job(v, True))
    for q in range(nd):
        for k in range(nm):
            synth.fill_device(v[f"m{q}_{k}"], segs,
                              synth.key(w.name, "micro_grad", q, k, w.t_first), *w.micro_grad)
    for fused in (False, True):
        ms = timed(lambda: job(v, fused), reps=3)
        if fused:
            nbytes = S * (nd * (6 + 10 * (nm - 2)) + 6 * nd + 26)
            desc = (f"accum1p3b job: {nd} ranks x {nm - 1} accumulate calls, then the step "
                    "folding in each rank's last micro-batch (6*N_d+26 B/elem)")
        else:
            nbytes = S * (nd * (6 + 10 * (nm - 2) + 8) + 2 * nd + 26)
            desc = (f"accum1p3b job: {nd} ranks x {nm} accumulate calls (last emits bf16), "
                    "then the step")
        record("accum_vec_kernel + step_vec_kernel" + (" (fused)" if fused else ""), desc,
               nbytes, ms)
    del v
    torch.cuda.empty_cache()
    return out


def next_rows(z, synth, w, L, holder, timed, placement):
    """The rows beyond the bf16 step, measured on llama8b-sized buffers:
    FSDP2 (dim-0) step, the step in bucket ranges, parameter gathers,
    re-cuts, fp32-contribution step and the step with the last micro-batch
    folded in.
    holder[0]: the bench's inputs (released here)."""
    import torch
    dev = torch.device("cuda:0")
    S, P = L.shard, L.padded
    hp = z.AdamW(**w.hp)
    out = []

    def row(name, kernel, desc, nbytes, ms):
        out.append({"row": name, "kernel": kernel, "workload": desc, "bytes_per_call": nbytes,
                    "ms": ms, "GBps": nbytes / (ms * 1e-3) / 1e9,
                    "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS})

    inp = holder.pop()
    # FSDP2 per-parameter layout, ZeRO-3 in place (COMPACT contributions)
    rows = [sh[1][0] for sh in w.shapes]
    Ld = z.Layout(w.numel, 0, w.n_d, w.rank, rows=rows)
    assert Ld.shard == S
    shard_out = inp.pout[:S]
    ms = timed(lambda: z.zero_shard_step(Ld, hp, 5, inp.grads, z.GRAD_COMPACT, *inp.state,
                                         shard_out, z.OUT_SHARD))
    row("fsdp2_step", "step_vec_kernel", "llama8b_fsdp2: Llama-3-8B per-parameter dim-0 "
        "layout, N_d=8, rank 7, in place", S * (2 * w.n_d + 26), ms)
    # the same layout with All-Gather slot output: every tensor's slice has
    # its own slot, so the step runs as table launches
    assert Ld.padded == P
    ms = timed(lambda: z.zero_shard_step(Ld, hp, 5, inp.grads, z.GRAD_COMPACT, *inp.state,
                                         inp.pout, z.OUT_AG_SLOT))
    row("fsdp2_step_slot", "step_table_kernel", "llama8b_fsdp2 with All-Gather slot output: "
        "291 per-tensor slots, 2 table launches", S * (2 * w.n_d + 26), ms)
    # ZeRO-2 stepping bucket by bucket (as each bucket's Reduce-Scatter
    # lands): the same update as one call per bucket range, captured in a
    # HIP graph so that the host's launch rate is not what is timed.  Single
    # buckets are also timed with the calls alternating between two streams
    # (the buckets are disjoint, so the order of their updates is free): one
    # call's ramp-up then overlaps the previous call's drain.
    nb = L.n_buckets
    for group, n_streams in ((1, 1), (1, 2), (32, 1)):
        def ranges(stream, side, group=group):
            for k, b0 in enumerate(range(0, nb, group)):
                st = side[k % len(side)] if side else stream
                z.zero_shard_step_buckets(L, hp, 6, b0, min(nb, b0 + group), inp.grads,
                                          z.GRAD_COMPACT, *inp.state, inp.pout, z.OUT_AG_SLOT,
                                          stream=st)
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        side = [torch.cuda.Stream() for _ in range(n_streams)] if n_streams > 1 else []
        with torch.cuda.stream(cap):
            with torch.cuda.graph(graph, stream=cap):
                for x in side:
                    x.wait_stream(cap)
                ranges(cap, side)
                for x in side:
                    cap.wait_stream(x)
        torch.cuda.current_stream().wait_stream(cap)
        ms = timed(graph.replay, reps=5)
        n_calls = (nb + group - 1) // group
        name = f"step_buckets_{group}" + ("_two_streams" if n_streams > 1 else "")
        row(name, "step_vec_kernel", f"llama8b step as {n_calls} calls of {group} bucket(s) "
            f"each on {n_streams} stream(s) (HIP graph)", S * (2 * w.n_d + 26), ms)
        del graph
    # All-Gather local part: the 8 bf16 shards (the contribution buffers
    # stand in for them) into the 8.03e9-element flat buffer
    ms = timed(lambda: z.zero_gather_params(L, inp.grads, inp.pout))
    row("gather", "gather_table_kernel", "llama8b: 8 rank shards -> 8,030,261,248-element flat "
        "buffer", 4 * P, ms)
    # the same two movements for the per-parameter (dim-0) layout: its
    # gather (one table launch per 48 tensors) and a re-cut of its bf16
    # shards for 4 bucketed ranks
    if Ld.padded <= inp.pout.numel():
        ms = timed(lambda: z.zero_gather_params(Ld, inp.grads, inp.pout[:Ld.padded]))
        row("gather_fsdp2", "gather_table_kernel", "llama8b_fsdp2: 8 rank shards -> "
            f"{Ld.padded:,}-element flat buffer", 4 * Ld.padded, ms)
    L4b = z.Layout(w.numel, w.cap, 4, 3)
    dst16 = torch.empty(L4b.shard, dtype=torch.int16, device=dev)
    ms = timed(lambda: z.zero_reshard(Ld, inp.grads, L4b, dst16), reps=5)
    row("reshard_fsdp2", "reshard_table_kernel<u16>", "llama8b bf16 params: 8 dim-0 shards -> "
        f"rank 3 of 4 bucketed ({L4b.shard} elements)", 4 * L4b.shard, ms)
    del inp, shard_out, dst16
    torch.cuda.empty_cache()
    # fp32 contributions
    inp, _ = make_inputs(z, synth, w, L, placement, grad_dtype=torch.float32, tune=MAIN_TUNE)
    ms = timed(lambda: z.zero_shard_step(L, hp, 7, inp.grads, z.GRAD_COMPACT, *inp.state,
                                         inp.pout, z.OUT_AG_SLOT))
    row("step_f32", "step_vec_kernel (fp32 contributions)", "llama8b with fp32 contributions "
        "(4*N_d+26 = 58 B/elem)", S * (4 * w.n_d + 26), ms)
    del inp
    torch.cuda.empty_cache()
    # the last no_sync micro-batch folded into the step: each rank's fp32
    # accumulator plus its bf16 micro-batch
    inp, _ = make_inputs(z, synth, w, L, placement, accumulators=True, grad_micro=1,
                         tune=MAIN_TUNE)
    ms = timed(lambda: z.zero_shard_step_accumulate(L, hp, 8, inp.accs, inp.grads, 0.25,
                                                    z.DTYPE_BF16, z.GRAD_COMPACT, *inp.state,
                                                    inp.pout, z.OUT_AG_SLOT))
    row("step_fused_accumulate", "step_vec_kernel (accumulator + last micro-batch)",
        "llama8b, each rank's contribution = bf16(acc + micro/4) inside the step "
        "(6*N_d+26 = 74 B/elem)", S * (6 * w.n_d + 26), ms)
    # re-cut one fp32 state array saved from 8 ranks for 4 ranks (the
    # accumulators stand in for the 8 saved shards)
    L4 = z.Layout(w.numel, w.cap, 4, 3)
    dst = torch.empty(L4.shard, dtype=torch.float32, device=dev)
    ms = timed(lambda: z.zero_reshard(L, inp.accs, L4, dst), reps=5)
    row("reshard", "reshard_kernel<u32>", "llama8b fp32 state: 8 ranks -> rank 3 of 4 "
        f"({L4.shard} elements)", 8 * L4.shard, ms)
    del inp, dst
    torch.cuda.empty_cache()
    return out


def all_configs(z, synth, workloads, steps, warmup, placement):
    """Step time of every shard workload (inputs resident, HIP events on the
    launch stream); FLAT workloads read their contributions from N_d padded
    flat buffers, the others from N_d shard-ordered buffers."""
    import torch
    stream = torch.cuda.current_stream()
    timed = make_timer(stream)
    res = []
    for name in workloads.NAMES + workloads.DIM0_NAMES:
        w = workloads.get(name)
        L = z.Layout(w.numel, w.cap, w.n_d, w.rank, rows=w.rows)
        S = L.shard
        inp, _ = make_inputs(z, synth, w, L, placement, tune=MAIN_TUNE)
        hp = z.AdamW(**w.hp)
        gl = z.GRAD_COMPACT if w.grad_layout == "compact" else z.GRAD_FLAT
        om = z.OUT_AG_SLOT if w.out_mode == "ag_slot" else z.OUT_SHARD

        def call():
            z.zero_shard_step(L, hp, w.t_first, inp.grads, gl, *inp.state, inp.pout, om)

        for _ in range(warmup):
            call()
        ms = timed(call, reps=steps)
        nbytes = S * (2 * w.n_d + 26)
        res.append({"workload": name, "shard_elems": S, "n_d": w.n_d, "buckets": L.n_buckets,
                    "grad_layout": w.grad_layout, "out_mode": w.out_mode,
                    "placement": placement, "ms": ms,
                    "Gelem_per_s": S / (ms * 1e-3) / 1e9, "GBps": nbytes / (ms * 1e-3) / 1e9,
                    "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS})
        if S < (1 << 24):
            # launch-bound sizes: 20 calls captured in one HIP graph, replayed
            side = torch.cuda.Stream()
            side.wait_stream(stream)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(side):
                with torch.cuda.graph(g, stream=side):
                    for _ in range(20):
                        z.zero_shard_step(L, hp, w.t_first, inp.grads, gl, *inp.state,
                                          inp.pout, om, stream=side)
            stream.wait_stream(side)
            torch.cuda.synchronize()
            gms = timed(g.replay, reps=5) / 20
            res[-1]["graph_ms"] = gms
            res[-1]["graph_GBps"] = nbytes / (gms * 1e-3) / 1e9
            del g
        print(f"# {name}: S={S} {ms:.4f} ms {res[-1]['GBps']:.0f} GB/s"
              + (f" (HIP graph of 20 calls: {res[-1]['graph_ms']:.4f} ms per call)"
                 if "graph_ms" in res[-1] else ""), file=sys.stderr, flush=True)
        del inp
        torch.cuda.empty_cache()
    return res


def time_steps(z, w, L, inp, steps, warmup, stream, launch=None):
    """Warmup, then `steps` timed calls of zero_shard_step on resident inputs
    (t advancing), each bracketed by HIP events on the launch stream; the
    whole timed region is also measured on the host clock, synchronised on
    both sides.  -> (host ms per step, per-call kernel ms list, next t)."""
    import torch
    hp = z.AdamW(**w.hp)
    gl = z.GRAD_COMPACT if w.grad_layout == "compact" else z.GRAD_FLAT
    om = z.OUT_AG_SLOT if w.out_mode == "ag_slot" else z.OUT_SHARD

    def step(t):
        z.zero_shard_step(L, hp, t, inp.grads, gl, *inp.state, inp.pout, om, launch=launch,
                          stream=stream)

    t = w.t_first
    for _ in range(warmup):
        step(t)
        t += 1
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        ev[k][0].record(stream)
        step(t)
        ev[k][1].record(stream)
        t += 1
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall * 1e3 / steps, [a.elapsed_time(b) for a, b in ev], t


def roofline_block(w, S, kernel_ms):
    """The step kernel's algorithmic bytes per launch over its average
    launch duration, against 8 TB/s; traffic from the committed counter
    summary when it was taken on the current kernel sources."""
    k_avg = sum(kernel_ms) / len(kernel_ms)
    alg_bytes = S * (2 * w.n_d + 26)
    achieved = alg_bytes / (k_avg * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBPS, "traffic": traffic_from_profiles(w.name, alg_bytes),
            "kernel": step_kernel_name(w.n_d, w.grad_layout == "flat" or w.out_mode == "ag_slot"),
            "kernel_avg_ms": k_avg, "kernel_median_ms": sorted(kernel_ms)[len(kernel_ms) // 2],
            "kernel_min_ms": min(kernel_ms), "algorithmic_bytes_per_launch": alg_bytes,
            "kernel_hash": kernel_hash()}


def placement_info(inp, searched_with="the same-mix probe (measure/stream_ceiling.hip)"):
    if inp.pool is None:
        return "separate", None
    if not inp.pool.tuning:
        return "pool", {"pool_GiB": inp.pool.nbytes / 2**30, "searched_with": None}
    return "tuned", {"pool_GiB": inp.pool.nbytes / 2**30,
                     "chosen_shift_GiB": inp.pool.shift / 2**30,
                     "searched_with": searched_with,
                     "ms_by_shift_GiB": [[sh / 2**30, ms] for sh, ms in inp.pool.tuning]}


def second_config(z, synth, name, args, stream):
    """One more full-size workload in the same run (its own buffers, freed
    afterwards): step time, roofline block and CPU oracle."""
    import torch
    w = workloads_mod().get(name)
    L = z.Layout(w.numel, w.cap, w.n_d, w.rank)
    S, P = L.shard, L.padded
    print(f"# workload {w.name}: S={S} P={P} N_d={w.n_d} buckets={L.n_buckets}", file=sys.stderr,
          flush=True)
    inp, segs = make_inputs(z, synth, w, L, args.placement, tune=MAIN_TUNE,
                            choose=mix_choose(L) if w.grad_layout == "compact" else None)
    used, tuning = placement_info(inp)
    ms_per_step, kernel_ms, _ = time_steps(z, w, L, inp, args.steps, args.warmup, stream)
    roof = roofline_block(w, S, kernel_ms)
    print(f"# {w.name}: {ms_per_step:.3f} ms/step wall, kernel avg {roof['kernel_avg_ms']:.3f} ms; "
          f"{roof['achieved']:.0f} GB/s ({100 * roof['frac']:.1f} % of 8 TB/s)", file=sys.stderr,
          flush=True)
    del inp
    torch.cuda.empty_cache()
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, segs, S, target_s=10.0)
    bpe = 2 * w.n_d + 26
    return {"workload": w.name, "description": WORKLOAD_LABEL[w.name], "shard_elems": S,
            "padded_elems": P, "n_d": w.n_d, "rank": w.rank, "buckets": L.n_buckets,
            "grad_layout": w.grad_layout, "out_mode": w.out_mode, "bytes_per_elem": bpe,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
            "value": S / (ms_per_step * 1e-3), "unit": "elem/s",
            "hbm_GBps": S * bpe / (ms_per_step * 1e-3) / 1e9,
            "hbm_frac_of_peak": S * bpe / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
            "placement": used, "placement_tuning": tuning, "roofline": roof, "cpu_baseline": cpu}


def placement_sweep(z, w, L, sweep, pool_gib=240, step_gib=8, reps=4):
    """Where the step's buffers sit in HBM, swept (printed as markdown).
    shifts: one large pool; the buffers laid out packed one after another,
    or by zero_placement_plan, and the whole arrangement moved through the
    pool in steps of step_gib.  poolsize: the planned arrangement at the
    start of pools of growing size.  Values are not initialised (timing
    only); every timed call is a whole shard step."""
    import torch
    from fsdp_sharded_optimizer_step_amd import binding
    from fsdp_sharded_optimizer_step_amd import placement as zp
    GiB = 1 << 30
    hp = z.AdamW(**w.hp)
    om = z.OUT_AG_SLOT if w.out_mode == "ag_slot" else z.OUT_SHARD
    gl = z.GRAD_COMPACT if w.grad_layout == "compact" else z.GRAD_FLAT
    specs = zp.step_specs(L, grad_layout=gl, out_mode=om)
    nbytes = [n * torch.empty((), dtype=dt).element_size() for _, n, dt, _ in specs]
    plan, need = binding.zero_placement_plan(nbytes, [sp[3] for sp in specs], zp.LANE_BYTES,
                                             zp.N_LANES, zp.ALIGN)
    packed, off = [], 0
    for n in nbytes:
        packed.append(off)
        off = (off + n + zp.ALIGN - 1) // zp.ALIGN * zp.ALIGN
    packed_need = off
    stream = torch.cuda.current_stream()
    timed = make_timer(stream)
    nd, bpe = L.n_d, 2 * L.n_d + 26

    def step_ms(pool, offs, shift):
        v = []
        for (_, _, dt, _), o, b in zip(specs, offs, nbytes):
            assert 0 <= o + shift and o + shift + b <= pool.numel()
            v.append(pool[o + shift:o + shift + b].view(dt))
        fn = lambda: z.zero_shard_step(L, hp, w.t_first, v[:nd], gl, v[nd], v[nd + 1],
                                       v[nd + 2], v[nd + 3], om)
        return min(timed(fn, reps=reps) for _ in range(2))

    print(f"workload {w.name}: S = {L.shard}, N_d = {nd}, {bpe} bytes per element; planned "
          f"arrangement {need / GiB:.1f} GiB, packed {packed_need / GiB:.1f} GiB; kernel "
          f"sources {kernel_hash()}\n")
    if sweep == "shifts":
        pool = torch.empty(pool_gib * GiB, dtype=torch.uint8, device="cuda:0")
        print(f"pool of {pool_gib} GiB; step ms (TB/s) with the arrangement shifted by:\n")
        print("| shift GiB | packed ms | packed TB/s | planned ms | planned TB/s |")
        print("|---|---|---|---|---|")
        last = min(pool_gib * GiB - need, pool_gib * GiB - packed_need)
        for sh in range(0, last // GiB + 1, step_gib):
            a = step_ms(pool, packed, sh * GiB)
            b = step_ms(pool, plan, sh * GiB)
            print(f"| {sh} | {a:.3f} | {L.shard * bpe / a / 1e9:.2f} | {b:.3f} | "
                  f"{L.shard * bpe / b / 1e9:.2f} |", flush=True)
    else:
        print("planned arrangement at the start of a pool of the plan's size + extra:\n")
        print("| extra GiB | pool GiB | step ms | TB/s |")
        print("|---|---|---|---|")
        for extra in range(0, 97, step_gib):
            pool = torch.empty(need + extra * GiB, dtype=torch.uint8, device="cuda:0")
            ms = step_ms(pool, plan, 0)
            print(f"| {extra} | {(need + extra * GiB) / GiB:.1f} | {ms:.3f} | "
                  f"{L.shard * bpe / ms / 1e9:.2f} |", flush=True)
            del pool
            torch.cuda.empty_cache()


def workloads_mod():
    from synth import workloads
    return workloads


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b", choices=sorted(WORKLOAD_LABEL))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-aux", action="store_true", help="skip the pack/accumulate timings")
    ap.add_argument("--no-more-configs", action="store_true",
                    help="time only --workload (by default the Llama-3-8B run also times the "
                         "two Llama-70B shards, N_d = 64, in the same JSON line)")
    ap.add_argument("--blocks", type=int, default=0)
    ap.add_argument("--threads", type=int, default=0)
    ap.add_argument("--placement", default="tuned",
                    choices=["tuned", "planned", "compact", "separate"],
                    help="tuned: the step's buffers in one pool laid out by zero_placement_plan, "
                         "its start chosen by timing the same-mix probe at a few shifts; "
                         "planned: the same pool at shift 0; compact: lanes just large enough "
                         "for the buffers, at shift 0; separate: one torch allocation per buffer")
    ap.add_argument("--all-configs", action="store_true",
                    help="time the step of every shard workload instead (one JSON line)")
    ap.add_argument("--placement-sweep", choices=["shifts", "poolsize"],
                    help="instead: time the step of --workload with its buffers at many places "
                         "in HBM (markdown table)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (3 times): the known-size "
                         "reference for scaling HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (the shard step of one rank); "
              "--gpus must be 1", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 1 << 30,
                          "copy_calibration_bytes_written": 1 << 30, "launches": 3}))
        return

    import fsdp_sharded_optimizer_step_amd as z
    import synth
    from synth import workloads

    z.load()
    if args.placement_sweep:
        w = workloads.get(args.workload)
        placement_sweep(z, w, z.Layout(w.numel, w.cap, w.n_d, w.rank), args.placement_sweep)
        return
    if args.all_configs:
        print(json.dumps({"per_config": all_configs(z, synth, workloads, args.steps,
                                                    args.warmup, args.placement)}), flush=True)
        return
    w = workloads.get(args.workload)
    L = z.Layout(w.numel, w.cap, w.n_d, w.rank)
    S, P = L.shard, L.padded
    print(f"# workload {w.name}: S={S} P={P} N_d={w.n_d} buckets={L.n_buckets}", file=sys.stderr,
          flush=True)
    inp, segs = make_inputs(z, synth, w, L, args.placement, tune=MAIN_TUNE,
                            choose=mix_choose(L) if w.grad_layout == "compact" else None)
    placement_used, tuning = placement_info(
        inp, "the same-mix probe (measure/stream_ceiling.hip)" if w.grad_layout == "compact"
        else "the step")
    if placement_used != "separate":
        placement_used = args.placement
    hp = z.AdamW(**w.hp)
    gl = z.GRAD_COMPACT if w.grad_layout == "compact" else z.GRAD_FLAT
    om = z.OUT_AG_SLOT if w.out_mode == "ag_slot" else z.OUT_SHARD
    launch = (args.blocks, args.threads, 0) if (args.blocks or args.threads) else None
    stream = torch.cuda.current_stream()
    ms_per_step, kernel_ms, t = time_steps(z, w, L, inp, args.steps, args.warmup, stream, launch)
    roof = roofline_block(w, S, kernel_ms)
    k_avg, achieved, alg_bytes = roof["kernel_avg_ms"], roof["achieved"], roof[
        "algorithmic_bytes_per_launch"]
    bytes_per_elem = 2 * w.n_d + 26
    print(f"# timed {args.steps} steps: {ms_per_step:.3f} ms/step wall, kernel avg {k_avg:.3f} ms "
          f"(min {min(kernel_ms):.3f}, max {max(kernel_ms):.3f}); {achieved:.0f} GB/s",
          file=sys.stderr, flush=True)
    # the same byte mix with trivial arithmetic, on the bench's own buffers
    # (after the timed region: it overwrites the state)
    import measure
    ceil_gbps, ceil_cfg = measure.stream_ceiling(inp.grads, inp.state, inp.pout, S)
    print(f"# same-mix streaming ceiling: {ceil_gbps:.0f} GB/s {ceil_cfg}", file=sys.stderr,
          flush=True)
    probes = measure.stream_probes(inp.grads, inp.state, inp.pout, S)
    print(f"# pure read {probes['read']['GBps']:.0f} GB/s, copy {probes['copy']['GBps']:.0f} GB/s "
          "on the same buffers", file=sys.stderr, flush=True)
    nxt = []
    holder = [inp]
    del inp
    if not args.no_aux and w.name == "llama8b":
        nxt = next_rows(z, synth, w, L, holder, make_timer(stream), args.placement)
    holder.clear()
    torch.cuda.empty_cache()
    # the same step on placements that need no timed search: one torch
    # allocation per buffer, the planned pool at its start, and a pool of
    # about 1.2x the buffers (lanes just large enough) at its start
    other = {}
    if not args.no_aux:
        for alt in ("separate", "planned", "compact"):
            inp, _ = make_inputs(z, synth, w, L, alt)
            ms_alt = make_timer(stream)(lambda: z.zero_shard_step(
                L, hp, t, inp.grads, gl, *inp.state, inp.pout, om), reps=10)
            work = sum(x.numel() * x.element_size() for x in inp.grads + inp.state + [inp.pout])
            other[alt] = {"kernel_avg_ms": ms_alt, "GBps": alg_bytes / (ms_alt * 1e-3) / 1e9,
                          "frac": alg_bytes / (ms_alt * 1e-3) / 1e9 / PEAK_HBM_GBPS,
                          "buffer_GiB": work / 2**30,
                          "pool_GiB": None if inp.pool is None else inp.pool.nbytes / 2**30}
            print(f"# placement {alt}: {ms_alt:.3f} ms, {other[alt]['GBps']:.0f} GB/s",
                  file=sys.stderr, flush=True)
            del inp
            torch.cuda.empty_cache()
    aux = nxt + ([] if args.no_aux else aux_kernels(z, synth, workloads, args.placement))
    for a in aux:
        print(f"# {a.get('row', a['kernel'])}: {a['ms']:.3f} ms, {a['GBps']:.0f} GB/s "
              f"({100 * a['frac']:.1f} % of 8 TB/s)", file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, segs, S)
    more = {}
    if w.name == "llama8b" and not args.no_more_configs:
        for name in ("llama70b", "llama70b_t"):
            more[name] = second_config(z, synth, name, args, stream)
    out = {
        "metric": "shard-step elements/s and achieved HBM GB/s (% of MI355X peak), 1 GPU",
        "value": S / (ms_per_step * 1e-3),
        "unit": "elem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded counter-based generator, resident in HBM)",
        "hbm_GBps": alg_bytes / (ms_per_step * 1e-3) / 1e9,
        "hbm_frac_of_peak": alg_bytes / (ms_per_step * 1e-3) / 1e9 / PEAK_HBM_GBPS,
        "config": {"workload": w.name, "description": WORKLOAD_LABEL[w.name], "shard_elems": S,
                   "padded_elems": P, "n_d": w.n_d, "rank": w.rank, "buckets": L.n_buckets,
                   "grad_layout": w.grad_layout, "out_mode": w.out_mode,
                   "bytes_per_elem": bytes_per_elem, "io": "bf16 grads and params, f32 state",
                   "placement": placement_used, "placement_tuning": tuning},
        "roofline": roof,
        "cpu_baseline": cpu,
        "configs": more,
        "same_mix_ceiling": {"GBps": ceil_gbps, "frac_of_peak": ceil_gbps / PEAK_HBM_GBPS,
                             "step_frac_of_ceiling": achieved / ceil_gbps,
                             "kernel": "measure/stream_ceiling.hip: the step's bytes, "
                                       "trivial arithmetic", "best_config": ceil_cfg,
                             "pure_read": probes["read"], "copy": probes["copy"]},
        "placement_comparison": other,
        "aux_kernels": aux,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
