"""Host-side checks of the binding and of the tensor queries, no GPU needed.

- zero_layout_tensor_flat: a tensor's range in the padded flat buffer equals
  where the oracle's pack puts that tensor's first and last elements.
- The Python wrappers refuse buffers shorter than the call reads or writes
  (the C ABI takes bare pointers and cannot see lengths) before touching the
  device: a host tensor of the right size gets past the size check and is
  then refused for not being on the GPU.
"""
import numpy as np
import pytest
import torch

import fsdp_sharded_optimizer_step_amd as z
import oracle
from synth import workloads


def _flat_ranges_from_pack(numel, cap, n_d, rows=None):
    """(first, last + 1) flat position of every non-empty tensor, read off
    the oracle's pack of tensors filled with their own stream positions."""
    pl = oracle.plan(numel, cap, n_d, rows=rows)
    off = np.concatenate([[0], np.cumsum(numel)])
    # value = stream position + 1, so 0 marks padding (Psi < 2^16 here)
    tens = [np.arange(off[t] + 1, off[t + 1] + 1, dtype=np.uint16) for t in range(len(numel))]
    flat = oracle.pack(tens, pl)
    out = {}
    for t in range(len(numel)):
        if numel[t]:
            first = np.flatnonzero(flat == off[t] + 1)
            last = np.flatnonzero(flat == off[t + 1])
            assert first.size == 1 and last.size == 1
            out[t] = (int(first[0]), int(last[0]) + 1)
    return pl, out


@pytest.mark.parametrize("seed", range(25))
def test_tensor_flat_range_equals_oracle_pack(seed):
    rng = np.random.default_rng(7000 + seed)
    n_t = int(rng.integers(1, 9))
    dim0 = seed % 3 == 0
    if dim0:
        rows = [int(v) for v in rng.integers(0, 30, n_t)]
        numel = [r * int(k) for r, k in zip(rows, rng.integers(1, 6, n_t))]
        cap = 0
    else:
        rows = None
        numel = [int(v) for v in rng.integers(0, 80, n_t)]
        cap = int(rng.choice([0, 1, 7, 16, 33, 100]))
    n_d = int(rng.choice([1, 2, 3, 4, 8]))
    pl, exp = _flat_ranges_from_pack(numel, cap, n_d, rows)
    L = z.Layout(numel, cap, n_d, n_d - 1, rows=rows)
    off = np.concatenate([[0], np.cumsum(numel)])
    for t in range(n_t):
        lo, hi = L.tensor_flat(t)
        if numel[t]:
            assert (lo, hi) == exp[t], (t, numel, cap, n_d)
        else:
            # an empty tensor: where it would start (the next real element's
            # flat position, or the end of the buffer)
            assert lo == hi
            later = [exp[u][0] for u in range(t + 1, n_t) if numel[u]]
            if rows is None:
                x = int(off[t])
                if x < sum(numel):
                    b = int(np.searchsorted(pl.stream_off, x, side="right") - 1)
                    assert lo == pl.padded_off[b] + (x - pl.stream_off[b])
                else:
                    assert lo == pl.padded_total
            else:
                assert lo == pl.padded_off[t]
            assert all(lo <= f for f in later)


@pytest.mark.parametrize("name", ["gpt2s", "llama8b", "llama70b_t", "gpt2s_fsdp2"])
def test_tensor_flat_range_on_workloads(name):
    """Closed forms on the workload lists: a tensor's first and last elements
    sit at their bucket's flat start plus their offset in the bucket."""
    w = workloads.get(name)
    pl = oracle.plan(w.numel, w.cap, w.n_d, rows=w.rows)
    L = z.Layout(w.numel, w.cap, w.n_d, w.rank, rows=w.rows)
    off = np.concatenate([[0], np.cumsum(w.numel)])

    def flat(x):
        b = int(np.searchsorted(pl.stream_off, x, side="right") - 1)
        return int(pl.padded_off[b] + (x - pl.stream_off[b]))

    for t in range(len(w.numel)):
        lo, hi = L.tensor_flat(t)
        if w.rows is not None:
            assert lo == pl.padded_off[t] and hi == lo + w.numel[t]
        else:
            assert (lo, hi) == (flat(off[t]), flat(off[t + 1] - 1) + 1)


def test_tensor_flat_errors():
    L = z.Layout([3, 4], 5, 2, 1)
    with pytest.raises(z.ZeroError):
        L.tensor_flat(2)
    with pytest.raises(z.ZeroError):
        L.tensor_flat(-1)


# ------------------------------------------------------------ buffer sizes
def _host(n, dtype):
    return torch.zeros(max(0, n), dtype=dtype)


def _raises_size(fn):
    with pytest.raises(ValueError, match="elements, the call needs at least"):
        fn()


def _raises_device(fn):
    with pytest.raises(ValueError, match="CUDA tensor"):
        fn()


@pytest.mark.parametrize("gl,om", [(z.GRAD_COMPACT, z.OUT_AG_SLOT), (z.GRAD_FLAT, z.OUT_SHARD),
                                   (z.GRAD_FLAT, z.OUT_AG_SLOT)])
def test_step_wrappers_refuse_short_buffers(gl, om):
    L = z.Layout([1000, 37, 500], 300, 4, 3)
    S, P = L.shard, L.padded
    ng = P if gl == z.GRAD_FLAT else S
    no = P if om == z.OUT_AG_SLOT else S
    hp = z.AdamW()

    def bufs(short=None):
        b = {"g": [_host(ng, torch.int16) for _ in range(4)],
             "gf": [_host(ng, torch.float32) for _ in range(4)],
             "acc": [_host(ng, torch.float32) for _ in range(4)],
             "master": _host(S, torch.float32), "m": _host(S, torch.float32),
             "v": _host(S, torch.float32), "p": _host(no, torch.int16),
             "rg": _host(S, torch.float32)}
        if short in ("g", "gf", "acc"):
            b[short][2] = _host(ng - 1, b[short][2].dtype)
        elif short:
            b[short] = _host(b[short].numel() - 1, b[short].dtype)
        return b

    def calls(b):
        return [
            lambda: z.zero_shard_step(L, hp, 1, b["g"], gl, b["master"], b["m"], b["v"], b["p"],
                                      om, b["rg"]),
            lambda: z.zero_shard_step(L, hp, 1, b["gf"], gl, b["master"], b["m"], b["v"], b["p"],
                                      om, b["rg"]),
            lambda: z.zero_shard_step_buckets(L, hp, 1, 0, L.n_buckets, b["g"], gl, b["master"],
                                              b["m"], b["v"], b["p"], om, b["rg"]),
            lambda: z.zero_shard_step_accumulate(L, hp, 1, b["acc"], b["g"], 0.25, z.DTYPE_BF16,
                                                 gl, b["master"], b["m"], b["v"], b["p"], om,
                                                 b["rg"]),
        ]

    for c in calls(bufs()):
        _raises_device(c)
    for short in ("master", "m", "v", "p", "rg"):
        for c in calls(bufs(short)):
            _raises_size(c)
    _raises_size(calls(bufs("g"))[0])
    _raises_size(calls(bufs("g"))[2])
    _raises_size(calls(bufs("g"))[3])
    _raises_size(calls(bufs("gf"))[1])
    _raises_size(calls(bufs("acc"))[3])


def test_accumulate_pack_gather_reshard_refuse_short_buffers():
    n = 1001
    acc, g, out = _host(n, torch.float32), _host(n, torch.int16), _host(n, torch.int16)
    _raises_device(lambda: z.zero_grad_accumulate(acc, g, 0.5, z.ACC_EMIT_BF16, out))
    _raises_size(lambda: z.zero_grad_accumulate(acc[:-1], g, 0.5, z.ACC_EMIT_BF16, out))
    _raises_size(lambda: z.zero_grad_accumulate(acc, g, 0.5, z.ACC_EMIT_BF16, out[:-1]))
    _raises_size(lambda: z.zero_grad_accumulate(acc, g, 0.5, 0, None, n=n + 1))

    numel = [1000, 37, 500]
    L = z.Layout(numel, 300, 4, 3)
    tens = [_host(k, torch.int16) for k in numel]
    flat = _host(L.padded, torch.int16)
    _raises_device(lambda: z.zero_bucket_pack(L, tens, flat))
    _raises_size(lambda: z.zero_bucket_pack(L, tens, flat[:-1]))
    _raises_size(lambda: z.zero_bucket_pack(L, tens[:1] + [tens[1][:-1]] + tens[2:], flat))

    shards = [_host(L.shard, torch.int16) for _ in range(4)]
    _raises_device(lambda: z.zero_gather_params(L, shards, flat))
    _raises_size(lambda: z.zero_gather_params(L, shards, flat[:-1]))
    _raises_size(lambda: z.zero_gather_params(L, shards[:3] + [shards[3][:-1]], flat))

    L2 = z.Layout(numel, 0, 2, 0)
    src = [_host(L.shard, torch.float32) for _ in range(4)]
    dst = _host(L2.shard, torch.float32)
    _raises_device(lambda: z.zero_reshard(L, src, L2, dst))
    _raises_size(lambda: z.zero_reshard(L, src, L2, dst[:-1]))
    _raises_size(lambda: z.zero_reshard(L, [src[0][:-1]] + src[1:], L2, dst))
