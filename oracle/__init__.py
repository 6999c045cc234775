"""ctypes wrapper around the CPU oracle (oracle/liboracle.so).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the product package.  Arguments are
numpy arrays (uint16 for bf16 bit patterns, float32 for state); this module
only marshals them.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_i64p = C.POINTER(C.c_int64)
_u16p = C.POINTER(C.c_uint16)
_f32p = C.POINTER(C.c_float)


class _Spec(C.Structure):
    _fields_ = [("numel", _i64p), ("rows", _i64p), ("n_tensors", C.c_int32), ("cap", C.c_int64),
                ("n_d", C.c_int32)]


_specp = C.POINTER(_Spec)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build_oracle
        build_oracle.build()
    lib = C.CDLL(_LIB_PATH)
    lib.oracle_round_bf16.argtypes = [_f32p, C.c_int64, _u16p]
    lib.oracle_round_bf16_patterns.argtypes = [C.c_uint64, C.c_uint64, _u16p]
    lib.oracle_plan_counts.argtypes = [_specp, _i64p, _i64p, _i64p]
    lib.oracle_plan_buckets.argtypes = [_specp] + [_i64p] * 5
    lib.oracle_plan_tensor_ranges.argtypes = [_specp, C.c_int32, _i64p, _i64p]
    lib.oracle_plan_map.argtypes = [_specp, C.c_int32, _i64p, C.c_int64, _i64p, _i64p]
    lib.oracle_pack.argtypes = [C.POINTER(_u16p), _specp, _u16p]
    lib.oracle_slice.argtypes = [_u16p, _specp, C.c_int32, _u16p]
    lib.oracle_gather.argtypes = [C.POINTER(_u16p), _specp, _u16p]
    lib.oracle_plan_locate.argtypes = [_specp, _i64p, C.c_int64, C.POINTER(C.c_int32), _i64p]
    lib.oracle_reshard.argtypes = [C.POINTER(C.c_void_p), _specp, _specp, C.c_int32, C.c_void_p,
                                   C.c_int32]
    lib.oracle_accumulate.argtypes = [_f32p, _u16p, C.c_int64, C.c_float, C.c_int32, C.c_int32,
                                      _u16p]
    lib.oracle_step_scalars.argtypes = [C.c_double] * 5 + [C.c_int64, _f32p]
    lib.oracle_shard_step.argtypes = [C.c_int32, C.POINTER(_u16p), C.c_int64] + [C.c_double] * 5 + [
        C.c_int64, _f32p, _f32p, _f32p, _u16p, _f32p, C.c_int32]
    lib.oracle_shard_step_f32.argtypes = [C.c_int32, C.POINTER(_f32p), C.c_int64] + [
        C.c_double] * 5 + [C.c_int64, _f32p, _f32p, _f32p, _u16p, _f32p, C.c_int32]
    lib.oracle_model_state_bytes.argtypes = [C.c_int32, C.c_int64, C.c_int64, C.c_int32]
    lib.oracle_model_state_bytes.restype = C.c_double
    lib.oracle_comm_bytes_per_gpu.argtypes = [C.c_int32, C.c_int64, C.c_int32]
    lib.oracle_comm_bytes_per_gpu.restype = C.c_double
    for name in ("oracle_plan_counts", "oracle_plan_buckets", "oracle_plan_tensor_ranges",
                 "oracle_plan_map", "oracle_pack", "oracle_slice", "oracle_gather",
                 "oracle_plan_locate", "oracle_reshard", "oracle_shard_step",
                 "oracle_shard_step_f32"):
        getattr(lib, name).restype = C.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, ct):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be contiguous"
    return a.ctypes.data_as(C.POINTER(ct))


def _i64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int64))


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: invalid arguments (rc={rc})")


# ----------------------------------------------------------------- cast
def round_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().oracle_round_bf16(_ptr(x, C.c_float), x.size, _ptr(out, C.c_uint16))
    return out


def round_bf16_patterns(lo: int, hi: int) -> np.ndarray:
    out = np.empty(hi - lo, dtype=np.uint16)
    _load().oracle_round_bf16_patterns(lo, hi, _ptr(out, C.c_uint16))
    return out


def widen_bf16(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------- layout
@dataclass
class Plan:
    numel: np.ndarray
    cap: int
    n_d: int
    n_buckets: int
    padded_total: int
    shard_len: int
    stream_off: np.ndarray
    len: np.ndarray
    padded_off: np.ndarray
    padded_len: np.ndarray
    shard_off: np.ndarray
    rows: np.ndarray | None = None

    def spec(self):
        return _make_spec(self.numel, self.rows, self.cap, self.n_d)

    def tensor_ranges(self, rank: int):
        n = self.numel.size
        lo = np.zeros(n, np.int64)
        hi = np.zeros(n, np.int64)
        _check(_load().oracle_plan_tensor_ranges(self.spec(), rank, _ptr(lo, C.c_int64),
                                                 _ptr(hi, C.c_int64)), "plan_tensor_ranges")
        return lo, hi

    def map(self, rank: int, idx):
        """shard indices -> (padded flat position, stream position or -1 for a pad)."""
        idx = _i64(idx)
        flat = np.empty(idx.size, np.int64)
        strm = np.empty(idx.size, np.int64)
        _check(_load().oracle_plan_map(self.spec(), rank, _ptr(idx, C.c_int64), idx.size,
                                       _ptr(flat, C.c_int64), _ptr(strm, C.c_int64)), "plan_map")
        return flat, strm


def _make_spec(numel, rows, cap, n_d):
    sp = _Spec(_ptr(numel, C.c_int64), _ptr(rows, C.c_int64) if rows is not None else None,
               numel.size, cap, n_d)
    sp._keep = (numel, rows)  # the arrays must outlive the struct
    return C.pointer(sp)


def plan(numel, cap: int, n_d: int, rows=None) -> Plan:
    """Bucketed flat layout (rows=None), or FSDP2 per-parameter dim-0 layout
    when `rows` gives each tensor's dim-0 size (cap is then ignored)."""
    numel = _i64(numel)
    rows = None if rows is None else _i64(rows)
    lib = _load()
    sp = _make_spec(numel, rows, cap, n_d)
    nb, pt, sl = C.c_int64(), C.c_int64(), C.c_int64()
    _check(lib.oracle_plan_counts(sp, C.byref(nb), C.byref(pt), C.byref(sl)), "plan_counts")
    arrs = [np.zeros(nb.value, np.int64) for _ in range(5)]
    _check(lib.oracle_plan_buckets(sp, *[_ptr(a, C.c_int64) for a in arrs]), "plan_buckets")
    return Plan(numel, cap, n_d, nb.value, pt.value, sl.value, *arrs, rows=rows)


# ----------------------------------------------------------------- pack / slice
def pack(tensors, pl: Plan) -> np.ndarray:
    ts = [np.ascontiguousarray(t, dtype=np.uint16).reshape(-1) for t in tensors]
    assert len(ts) == pl.numel.size and all(t.size == n for t, n in zip(ts, pl.numel))
    arr = (_u16p * max(1, len(ts)))(*[_ptr(t, C.c_uint16) for t in ts])
    out = np.empty(pl.padded_total, np.uint16)
    _check(_load().oracle_pack(arr, pl.spec(), _ptr(out, C.c_uint16)), "pack")
    return out


def slice_shard(flat: np.ndarray, pl: Plan, rank: int) -> np.ndarray:
    flat = np.ascontiguousarray(flat, dtype=np.uint16)
    assert flat.size == pl.padded_total
    out = np.empty(pl.shard_len, np.uint16)
    _check(_load().oracle_slice(_ptr(flat, C.c_uint16), pl.spec(), rank, _ptr(out, C.c_uint16)),
           "slice")
    return out


def gather(shards, pl: Plan) -> np.ndarray:
    """The N_d ranks' shards -> the padded flat buffer (local All-Gather)."""
    ss = [np.ascontiguousarray(x, dtype=np.uint16).reshape(-1) for x in shards]
    assert len(ss) == pl.n_d and all(x.size == pl.shard_len for x in ss)
    arr = (_u16p * len(ss))(*[_ptr(x, C.c_uint16) for x in ss])
    out = np.empty(pl.padded_total, np.uint16)
    _check(_load().oracle_gather(arr, pl.spec(), _ptr(out, C.c_uint16)), "gather")
    return out


def locate(pl: Plan, xs):
    """stream positions -> (owning rank, index in its shard)"""
    xs = _i64(xs)
    r = np.empty(xs.size, np.int32)
    i = np.empty(xs.size, np.int64)
    _check(_load().oracle_plan_locate(pl.spec(), _ptr(xs, C.c_int64), xs.size,
                                      _ptr(r, C.c_int32), _ptr(i, C.c_int64)), "plan_locate")
    return r, i


def reshard(src_shards, src: Plan, dst: Plan, dst_rank: int) -> np.ndarray:
    """Re-cut one per-element array from src's shards to dst's shard of rank dst_rank."""
    ss = [np.ascontiguousarray(x) for x in src_shards]
    dt = ss[0].dtype
    assert dt in (np.float32, np.uint16) and all(x.dtype == dt for x in ss)
    assert np.array_equal(src.numel, dst.numel) and len(ss) == src.n_d
    arr = (C.c_void_p * len(ss))(*[x.ctypes.data for x in ss])
    out = np.empty(dst.shard_len, dt)
    _check(_load().oracle_reshard(arr, src.spec(), dst.spec(), dst_rank, out.ctypes.data,
                                  dt.itemsize), "reshard")
    return out


# ----------------------------------------------------------------- accumulate
def accumulate(acc: np.ndarray, g: np.ndarray, scale: float, overwrite: bool,
               store_acc: bool = True, emit: bool = False):
    """In-place on `acc`; returns the emitted bf16 array (or None)."""
    assert acc.dtype == np.float32 and acc.flags["C_CONTIGUOUS"]
    g = np.ascontiguousarray(g, dtype=np.uint16)
    assert g.size == acc.size
    out = np.empty(acc.size, np.uint16) if emit else None
    _load().oracle_accumulate(_ptr(acc, C.c_float), _ptr(g, C.c_uint16), acc.size, scale,
                              int(overwrite), int(store_acc),
                              _ptr(out, C.c_uint16) if emit else None)
    return out


# ----------------------------------------------------------------- step
@dataclass
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1


def step_scalars(hp: AdamW, t: int) -> np.ndarray:
    out = np.zeros(8, np.float32)
    _load().oracle_step_scalars(hp.lr, hp.beta1, hp.beta2, hp.eps, hp.weight_decay, t,
                                _ptr(out, C.c_float))
    return out


def shard_step(grads, master, m, v, hp: AdamW, t: int, want_grad: bool = False,
               nthreads: int = 1):
    """One reduce + AdamW + cast over a shard, in place on master/m/v.

    grads: list of n_d uint16 arrays (contributions in shard order).
    Returns (p_bf16, g_avg or None).
    """
    gs = [np.ascontiguousarray(g, dtype=np.uint16).reshape(-1) for g in grads]
    n = master.size
    for a in (master, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"] and a.size == n
    assert all(g.size == n for g in gs)
    arr = (_u16p * len(gs))(*[_ptr(g, C.c_uint16) for g in gs])
    p = np.empty(n, np.uint16)
    g_out = np.empty(n, np.float32) if want_grad else None
    _check(_load().oracle_shard_step(len(gs), arr, n, hp.lr, hp.beta1, hp.beta2, hp.eps,
                                     hp.weight_decay, t, _ptr(master, C.c_float),
                                     _ptr(m, C.c_float), _ptr(v, C.c_float), _ptr(p, C.c_uint16),
                                     _ptr(g_out, C.c_float) if want_grad else None, nthreads),
           "shard_step")
    return p, g_out


def shard_step_f32(grads, master, m, v, hp: AdamW, t: int, want_grad: bool = False,
                   nthreads: int = 1):
    """As shard_step, with binary32 contributions."""
    gs = [np.ascontiguousarray(g, dtype=np.float32).reshape(-1) for g in grads]
    n = master.size
    for a in (master, m, v):
        assert a.dtype == np.float32 and a.flags["C_CONTIGUOUS"] and a.size == n
    assert all(g.size == n for g in gs)
    arr = (_f32p * len(gs))(*[_ptr(g, C.c_float) for g in gs])
    p = np.empty(n, np.uint16)
    g_out = np.empty(n, np.float32) if want_grad else None
    _check(_load().oracle_shard_step_f32(len(gs), arr, n, hp.lr, hp.beta1, hp.beta2, hp.eps,
                                         hp.weight_decay, t, _ptr(master, C.c_float),
                                         _ptr(m, C.c_float), _ptr(v, C.c_float),
                                         _ptr(p, C.c_uint16),
                                         _ptr(g_out, C.c_float) if want_grad else None, nthreads),
           "shard_step_f32")
    return p, g_out


# ----------------------------------------------------------------- accounting
MODES = {"baseline": 0, "zero1": 1, "zero2": 2, "zero3": 3}


def model_state_bytes(mode: str, P: int, S: int, k: int = 12) -> float:
    return _load().oracle_model_state_bytes(MODES[mode], P, S, k)


COMM_MODES = {"ddp": 0, "zero1": 1, "zero2": 2, "zero3": 3}


def comm_bytes_per_gpu(mode: str, P: int, n_d: int) -> float:
    """Bytes one GPU sends per training step under the ring model (16-bit
    parameters and gradients over a P-element padded layout)."""
    return _load().oracle_comm_bytes_per_gpu(COMM_MODES[mode], P, n_d)
