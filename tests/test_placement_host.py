"""The placement pool's host logic on CPU memory: views carved from one pool
at the planner's offsets, the spare-room shift chosen by the timing callback,
and the step's buffer specs."""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_step_amd as z
from fsdp_sharded_optimizer_step_amd import placement as zp

MiB = 1 << 20


def _spans(pool):
    return sorted((pool.offsets[n], pool.offsets[n] + v.numel() * v.element_size())
                  for n, v in pool.views.items())


def test_pool_views_are_disjoint_typed_and_at_the_plan_offsets():
    specs = [("a", 1000, torch.float32, 8.0), ("b", 3000, torch.int16, 2.0),
             ("c", 10, torch.float32, 8.0), ("d", 70000, torch.int16, 2.0)]
    pool = zp.Pool(specs, device="cpu", lane_bytes=MiB, n_lanes=3, align=256)
    spans = _spans(pool)
    assert all(a[1] <= b[0] for a, b in zip(spans, spans[1:]))
    base = pool.buf.data_ptr()
    for name, n, dt, _ in specs:
        v = pool[name]
        assert v.dtype == dt and v.numel() == n
        assert v.data_ptr() - base == pool.offsets[name]
        assert pool.offsets[name] % 256 == 0
    # the two heavy buffers go to different lanes
    assert pool.offsets["a"] // MiB % 3 != pool.offsets["c"] // MiB % 3
    # writing one view leaves the others untouched
    pool["b"].fill_(7)
    assert int(pool["a"].abs().sum()) == 0 and int(pool["d"].abs().sum()) == 0


def test_pool_shift_is_chosen_by_the_callback():
    """Spare room of 4 MiB, candidates every 1 MiB: the callback sees the views
    at each candidate shift and the fastest (lowest) one is kept."""
    specs = [("x", 4096, torch.float32, 8.0), ("y", 4096, torch.int16, 2.0)]
    plain = zp.Pool(specs, device="cpu", lane_bytes=MiB, n_lanes=3, align=256)
    seen = []

    def choose(views):
        seen.append(views["x"].data_ptr())
        return abs(len(seen) - 3) + 1.0   # the third candidate (2 MiB) is the fastest

    pool = zp.Pool(specs, device="cpu", lane_bytes=MiB, n_lanes=3, align=256, slack=4 * MiB,
                   choose=choose, shift_step=MiB)
    assert [sh for sh, _ in pool.tuning] == [0, MiB, 2 * MiB, 3 * MiB, 4 * MiB]
    assert [p - seen[0] for p in seen] == [0, MiB, 2 * MiB, 3 * MiB, 4 * MiB]
    assert pool.shift == 2 * MiB
    assert pool.offsets["x"] == plain.offsets["x"] + 2 * MiB
    assert pool["x"].data_ptr() - pool.buf.data_ptr() == pool.offsets["x"]
    assert pool.nbytes == plain.nbytes + 4 * MiB


def test_step_specs_follow_the_layout_and_modes():
    L = z.Layout([1000, 37, 4096, 3], 1500, 4, 3)
    specs = {s[0]: s for s in zp.step_specs(L, grad_layout=z.GRAD_FLAT, out_mode=z.OUT_AG_SLOT,
                                             reduced_grad=True)}
    assert all(specs[f"g{q}"][1] == L.padded and specs[f"g{q}"][3] == 2 for q in range(4))
    assert specs["master"][1] == L.shard and specs["master"][3] == 8
    assert specs["param_out"][1] == L.padded and specs["reduced_grad"][1] == L.shard
    specs = {s[0]: s for s in zp.step_specs(L, grad_dtype=torch.float32,
                                             grad_layout=z.GRAD_COMPACT, out_mode=z.OUT_SHARD,
                                             accumulators=True)}
    assert specs["g0"][1] == L.shard and specs["g0"][2] == torch.float32 and specs["g0"][3] == 4
    assert specs["a3"][2] == torch.float32 and specs["param_out"][1] == L.shard
    assert "reduced_grad" not in specs


def test_pool_rejects_bad_plans():
    with pytest.raises(z.ZeroError):
        zp.Pool([("x", 10, torch.float32, 1.0)], device="cpu", lane_bytes=1000, align=256)
    with pytest.raises(z.ZeroError):
        zp.Pool([("x", 10, torch.float32, float("nan"))], device="cpu", lane_bytes=MiB)
