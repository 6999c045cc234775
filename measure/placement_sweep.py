"""Placement sweeps of the shard step's buffers (measurement infrastructure).

The same buffers, stepped by the same kernel, run at different speeds
depending on where they sit in HBM.  Two sweeps, printed as markdown:

  shifts    one large pool; the step's 12 buffers (N_d contributions,
            master, m, v, output) laid out either packed one after another
            or by zero_placement_plan, and the whole arrangement moved
            through the pool in steps of --step-gib
  poolsize  the planned arrangement at the start of pools of growing size

Usage (one GPU):  python measure/placement_sweep.py shifts
                  python measure/placement_sweep.py poolsize
Values are not initialised (timing only).
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

GiB, MiB = 1 << 30, 1 << 20


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("sweep", choices=["shifts", "poolsize"])
    ap.add_argument("--workload", default="llama8b")
    ap.add_argument("--pool-gib", type=int, default=240)
    ap.add_argument("--step-gib", type=int, default=8)
    ap.add_argument("--reps", type=int, default=4)
    args = ap.parse_args()

    import torch
    import fsdp_sharded_optimizer_step_amd as z
    from fsdp_sharded_optimizer_step_amd import binding
    from fsdp_sharded_optimizer_step_amd import placement as zp
    from synth import workloads

    w = workloads.get(args.workload)
    L = z.Layout(w.numel, w.cap, w.n_d, w.rank)
    hp = z.AdamW(**w.hp)
    om = z.OUT_AG_SLOT if w.out_mode == "ag_slot" else z.OUT_SHARD
    gl = z.GRAD_COMPACT if w.grad_layout == "compact" else z.GRAD_FLAT
    specs = zp.step_specs(L, grad_layout=gl, out_mode=om)
    esz = [torch.empty((), dtype=dt).element_size() for _, _, dt, _ in specs]
    nbytes = [n * e for (_, n, _, _), e in zip(specs, esz)]
    plan, need = binding.zero_placement_plan(nbytes, [s[3] for s in specs], zp.LANE_BYTES,
                                             zp.N_LANES, zp.ALIGN)
    packed, off = [], 0
    for n in nbytes:
        packed.append(off)
        off = (off + n + zp.ALIGN - 1) // zp.ALIGN * zp.ALIGN
    packed_need = off
    stream = torch.cuda.current_stream()
    nd = L.n_d
    bpe = 2 * nd + 26

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(2):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(args.reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / args.reps
            best = ms if best is None else min(best, ms)
        return best

    def step_ms(pool, offs, shift):
        v = []
        for (name, n, dt, _), o, b in zip(specs, offs, nbytes):
            assert 0 <= o + shift and o + shift + b <= pool.numel()
            v.append(pool[o + shift:o + shift + b].view(dt))
        return timed(lambda: z.zero_shard_step(L, hp, w.t_first, v[:nd], gl, v[nd], v[nd + 1],
                                               v[nd + 2], v[nd + 3], om))

    print(f"workload {w.name}: S = {L.shard}, N_d = {nd}, {bpe} bytes per element; "
          f"planned arrangement {need / GiB:.1f} GiB, packed {packed_need / GiB:.1f} GiB\n")
    if args.sweep == "shifts":
        pool = torch.empty(args.pool_gib * GiB, dtype=torch.uint8, device="cuda:0")
        print(f"pool of {args.pool_gib} GiB; step ms (TB/s) with the arrangement shifted by:\n")
        print("| shift GiB | packed ms | packed TB/s | planned ms | planned TB/s |")
        print("|---|---|---|---|---|")
        last = min(args.pool_gib * GiB - need, args.pool_gib * GiB - packed_need)
        for sh in range(0, last // GiB + 1, args.step_gib):
            a = step_ms(pool, packed, sh * GiB)
            b = step_ms(pool, plan, sh * GiB)
            print(f"| {sh} | {a:.3f} | {L.shard * bpe / a / 1e9:.2f} | {b:.3f} | "
                  f"{L.shard * bpe / b / 1e9:.2f} |", flush=True)
    else:
        print("planned arrangement at the start of a pool of the plan's size + extra:\n")
        print("| extra GiB | pool GiB | step ms | TB/s |")
        print("|---|---|---|---|")
        for extra in range(0, 97, args.step_gib):
            pool = torch.empty(need + extra * GiB, dtype=torch.uint8, device="cuda:0")
            ms = step_ms(pool, plan, 0)
            print(f"| {extra} | {(need + extra * GiB) / GiB:.1f} | {ms:.3f} | "
                  f"{L.shard * bpe / ms / 1e9:.2f} |", flush=True)
            del pool
            torch.cuda.empty_cache()


if __name__ == "__main__":
    main()
