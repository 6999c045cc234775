"""Thin Python binding of libzero_shard.so (the C ABI in include/zero_shard.h).

Argument marshalling only: torch CUDA tensors supply device pointers and the
current HIP stream; every step of the update runs in the library's kernels.
bf16 buffers may be torch.bfloat16, torch.int16 or torch.uint16 tensors (the
library reads and writes 16-bit patterns).  Failing to find the built library
raises; there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libzero_shard.so")

ZERO_OK, ZERO_EINVAL, ZERO_ERANGE, ZERO_EHIP, ZERO_EOVERLAP = 0, -1, -3, -4, -5
ZERO_MAX_ND = 256
ZERO_MAX_ND_FUSED = 128
GRAD_COMPACT, GRAD_FLAT = 0, 1
OUT_AG_SLOT, OUT_SHARD = 0, 1
ACC_OVERWRITE, ACC_EMIT_BF16, ACC_NO_STORE = 1, 2, 4

EXPORTS = ("zero_layout_create", "zero_layout_destroy", "zero_layout_psi", "zero_layout_padded",
           "zero_layout_shard", "zero_layout_n_buckets", "zero_layout_n_d", "zero_layout_rank",
           "zero_layout_bucket", "zero_layout_tensor", "zero_bucket_pack", "zero_grad_accumulate",
           "zero_shard_step", "zero_shard_step_ex", "zero_step_scalars", "zero_strerror",
           "zero_gather_params", "zero_reshard", "zero_layout_create_dim0", "zero_layout_kind",
           "zero_shard_step_accumulate", "zero_placement_plan", "zero_shard_step_buckets",
           "zero_layout_tensor_flat")


class ZeroError(RuntimeError):
    def __init__(self, where: str, status: int):
        super().__init__(f"{where}: {_lib_strerror(status)} (status {status})")
        self.status = status


class _AdamW(C.Structure):
    _fields_ = [("lr", C.c_double), ("beta1", C.c_double), ("beta2", C.c_double),
                ("eps", C.c_double), ("weight_decay", C.c_double)]


DTYPE_BF16, DTYPE_F32 = 0, 1


class _Options(C.Structure):
    _fields_ = [("grad_dtype", C.c_int32), ("blocks", C.c_int32), ("threads", C.c_int32),
                ("path", C.c_int32)]


_lib = None
_i64p = C.POINTER(C.c_int64)


def load():
    """Load the built library (raises if it is missing)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                           "(no fallback path exists)")
    lib = C.CDLL(LIB_PATH)
    vp = C.c_void_p
    lib.zero_layout_create.argtypes = [_i64p, C.c_int32, C.c_int64, C.c_int32, C.c_int32,
                                       C.POINTER(vp)]
    lib.zero_layout_create_dim0.argtypes = [_i64p, _i64p, C.c_int32, C.c_int32, C.c_int32,
                                            C.POINTER(vp)]
    lib.zero_layout_kind.argtypes = [vp]
    lib.zero_layout_kind.restype = C.c_int32
    lib.zero_layout_destroy.argtypes = [vp]
    lib.zero_layout_destroy.restype = None
    for name in ("zero_layout_psi", "zero_layout_padded", "zero_layout_shard",
                 "zero_layout_n_buckets"):
        getattr(lib, name).argtypes = [vp]
        getattr(lib, name).restype = C.c_int64
    for name in ("zero_layout_n_d", "zero_layout_rank"):
        getattr(lib, name).argtypes = [vp]
        getattr(lib, name).restype = C.c_int32
    lib.zero_layout_bucket.argtypes = [vp, C.c_int64] + [_i64p] * 5
    lib.zero_layout_tensor.argtypes = [vp, C.c_int32] + [_i64p] * 3
    lib.zero_layout_tensor_flat.argtypes = [vp, C.c_int32] + [_i64p] * 2
    lib.zero_bucket_pack.argtypes = [vp, C.POINTER(vp), C.c_int64, C.c_int64, vp, vp]
    lib.zero_grad_accumulate.argtypes = [vp, vp, C.c_int64, C.c_float, C.c_uint32, vp, vp]
    lib.zero_shard_step.argtypes = [vp, C.POINTER(_AdamW), C.c_int64, C.POINTER(vp), C.c_int32,
                                    vp, vp, vp, vp, C.c_int32, vp, vp]
    lib.zero_shard_step_ex.argtypes = [vp, C.POINTER(_AdamW), C.c_int64, C.POINTER(vp),
                                       C.c_int32, vp, vp, vp, vp, C.c_int32, vp,
                                       C.POINTER(_Options), vp]
    lib.zero_shard_step_buckets.argtypes = [vp, C.POINTER(_AdamW), C.c_int64, C.c_int64,
                                            C.c_int64, C.POINTER(vp), C.c_int32, vp, vp, vp,
                                            vp, C.c_int32, vp, C.POINTER(_Options), vp]
    lib.zero_shard_step_accumulate.argtypes = [vp, C.POINTER(_AdamW), C.c_int64, C.POINTER(vp),
                                               C.POINTER(vp), C.c_float, C.c_int32, C.c_int32,
                                               vp, vp, vp, vp, C.c_int32, vp,
                                               C.POINTER(_Options), vp]
    lib.zero_gather_params.argtypes = [vp, C.POINTER(vp), C.c_int64, C.c_int64, vp, vp]
    lib.zero_reshard.argtypes = [vp, C.POINTER(vp), vp, vp, C.c_int32, vp]
    lib.zero_step_scalars.argtypes = [C.POINTER(_AdamW), C.c_int64, C.POINTER(C.c_float)]
    lib.zero_placement_plan.argtypes = [C.c_int32, _i64p, C.POINTER(C.c_double), C.c_int64,
                                        C.c_int32, C.c_int64, _i64p, _i64p]
    lib.zero_strerror.argtypes = [C.c_int]
    lib.zero_strerror.restype = C.c_char_p
    _lib = lib
    return lib


def _lib_strerror(status: int) -> str:
    try:
        return load().zero_strerror(status).decode()
    except Exception:  # pragma: no cover - only used for messages
        return "error"


def _check(where: str, rc: int):
    if rc != ZERO_OK:
        raise ZeroError(where, rc)


@dataclass
class AdamW:
    lr: float = 1e-3
    beta1: float = 0.9
    beta2: float = 0.95
    eps: float = 1e-8
    weight_decay: float = 0.1

    def _c(self):
        return _AdamW(self.lr, self.beta1, self.beta2, self.eps, self.weight_decay)


class Layout:
    """Owning wrapper of a zero_layout (host object)."""

    def __init__(self, numel, bucket_cap: int, n_d: int, rank: int, rows=None):
        """Bucketed flat layout; with `rows` (each tensor's dim-0 size) the
        per-parameter dim-0 layout instead (bucket_cap is then unused)."""
        lib = load()
        arr = (C.c_int64 * max(1, len(numel)))(*[int(n) for n in numel])
        h = C.c_void_p()
        if rows is None:
            _check("zero_layout_create", lib.zero_layout_create(
                arr, len(numel), int(bucket_cap), int(n_d), int(rank), C.byref(h)))
        else:
            rarr = (C.c_int64 * max(1, len(rows)))(*[int(r) for r in rows])
            _check("zero_layout_create_dim0", lib.zero_layout_create_dim0(
                arr, rarr, len(numel), int(n_d), int(rank), C.byref(h)))
        self._h = h
        self.n_tensors = len(numel)
        self.numel = [int(n) for n in numel]

    @property
    def handle(self):
        return self._h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.zero_layout_destroy(h)
            self._h = None

    psi = property(lambda self: load().zero_layout_psi(self._h))
    padded = property(lambda self: load().zero_layout_padded(self._h))
    shard = property(lambda self: load().zero_layout_shard(self._h))
    n_buckets = property(lambda self: load().zero_layout_n_buckets(self._h))
    n_d = property(lambda self: load().zero_layout_n_d(self._h))
    rank = property(lambda self: load().zero_layout_rank(self._h))
    kind = property(lambda self: load().zero_layout_kind(self._h))

    def bucket(self, b: int):
        """-> (stream_off, len, padded_off, padded_len, shard_off)"""
        vals = [C.c_int64() for _ in range(5)]
        _check("zero_layout_bucket", load().zero_layout_bucket(self._h, b, *[C.byref(v) for v in vals]))
        return tuple(v.value for v in vals)

    def buckets(self):
        return [self.bucket(b) for b in range(self.n_buckets)]

    def tensor(self, t: int):
        """-> (stream_off, shard_lo, shard_hi)"""
        vals = [C.c_int64() for _ in range(3)]
        _check("zero_layout_tensor", load().zero_layout_tensor(self._h, t, *[C.byref(v) for v in vals]))
        return tuple(v.value for v in vals)

    def tensor_flat(self, t: int):
        """-> (flat_lo, flat_hi): tensor t's range in the padded flat buffer"""
        vals = [C.c_int64() for _ in range(2)]
        _check("zero_layout_tensor_flat",
               load().zero_layout_tensor_flat(self._h, t, *[C.byref(v) for v in vals]))
        return tuple(v.value for v in vals)


def _stream_ptr(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _need(t, name, n):
    """The C ABI receives bare pointers and cannot know buffer lengths: a
    tensor shorter than what the call reads or writes would become an
    out-of-bounds device access, so it is refused here (before the dtype and
    device checks, so the check also runs on a host without a GPU)."""
    if t is not None and n is not None and t.numel() < n:
        raise ValueError(f"{name}: has {t.numel()} elements, the call needs at least {n}")


def _dev16(t, name, n=None):
    if t is None:
        return None
    _need(t, name, n)
    if not (t.is_cuda and t.is_contiguous() and t.element_size() == 2):
        raise ValueError(f"{name}: needs a contiguous 16-bit CUDA tensor")
    return C.c_void_p(t.data_ptr())


def _dev32(t, name, n=None):
    import torch
    if t is None:
        return None
    _need(t, name, n)
    if not (t.is_cuda and t.is_contiguous() and t.dtype == torch.float32):
        raise ValueError(f"{name}: needs a contiguous float32 CUDA tensor")
    return C.c_void_p(t.data_ptr())


def _ptr_array(tensors, name, check=None, n=None):
    """Host array of device pointers; `n`: the elements each entry must hold
    (an int for all, or a list with one entry per tensor)."""
    check = check or _dev16
    arr = (C.c_void_p * max(1, len(tensors)))()
    for k, t in enumerate(tensors):
        nk = n[k] if isinstance(n, (list, tuple)) else n
        arr[k] = None if t is None else check(t, f"{name}[{k}]", nk).value
    return arr


def _sizes(*items):
    """(tensor or list of tensors, name, elements needed) for every buffer
    of a call, checked before any pointer is marshalled."""
    for ts, name, n in items:
        if isinstance(ts, (list, tuple)):
            for k, t in enumerate(ts):
                _need(t, f"{name}[{k}]", n[k] if isinstance(n, (list, tuple)) else n)
        else:
            _need(ts, name, n)


def _step_sizes(layout: Layout, grad_layout: int, out_mode: int):
    """(elements per contribution, per state array, of the parameter output)
    of a step call on `layout`."""
    S, P = layout.shard, layout.padded
    return (P if grad_layout == GRAD_FLAT else S), S, (P if out_mode == OUT_AG_SLOT else S)


def zero_bucket_pack(layout: Layout, tensor_grads, flat_out, bucket_begin: int = 0,
                     bucket_end: int | None = None, stream=None):
    if len(tensor_grads) != layout.n_tensors:
        raise ValueError("zero_bucket_pack: one pointer per tensor is required")
    end = layout.n_buckets if bucket_end is None else bucket_end
    _sizes((tensor_grads, "tensor_grads", layout.numel), (flat_out, "flat_out", layout.padded))
    _check("zero_bucket_pack", load().zero_bucket_pack(
        layout.handle, _ptr_array(tensor_grads, "tensor_grads", n=layout.numel), bucket_begin,
        end, _dev16(flat_out, "flat_out", layout.padded), _stream_ptr(stream)))


def zero_grad_accumulate(acc, grad, scale: float, flags: int = 0, bf16_out=None, n=None,
                         stream=None):
    n = grad.numel() if n is None else int(n)
    _sizes((acc, "acc", n), (grad, "grad", n), (bf16_out, "bf16_out", n))
    _check("zero_grad_accumulate", load().zero_grad_accumulate(
        _dev32(acc, "acc", n), _dev16(grad, "grad", n), n, scale, flags,
        _dev16(bf16_out, "bf16_out", n), _stream_ptr(stream)))


def zero_shard_step(layout: Layout, hp: AdamW, t: int, rank_grads, grad_layout: int, master,
                    exp_avg, exp_avg_sq, param_out, out_mode: int, reduced_grad_out=None,
                    stream=None, launch=None):
    """One shard step.  bf16 contributions (16-bit tensors) go through
    zero_shard_step; float32 contributions, or an explicit launch shape
    `launch` = (blocks, threads, path), through zero_shard_step_ex."""
    import torch
    if len(rank_grads) != layout.n_d:
        raise ValueError("zero_shard_step: one contribution per rank is required")
    f32 = len(rank_grads) > 0 and rank_grads[0] is not None and rank_grads[0].dtype == torch.float32
    ng, ns, no = _step_sizes(layout, grad_layout, out_mode)
    _sizes((rank_grads, "rank_grads", ng), (master, "master", ns), (exp_avg, "exp_avg", ns),
           (exp_avg_sq, "exp_avg_sq", ns), (param_out, "param_out", no),
           (reduced_grad_out, "reduced_grad_out", ns))
    grads = _ptr_array(rank_grads, "rank_grads", _dev32 if f32 else _dev16, ng)
    args = [layout.handle, C.byref(hp._c()), int(t), grads, grad_layout,
            _dev32(master, "master", ns), _dev32(exp_avg, "exp_avg", ns),
            _dev32(exp_avg_sq, "exp_avg_sq", ns), _dev16(param_out, "param_out", no), out_mode,
            _dev32(reduced_grad_out, "reduced_grad_out", ns)]
    if launch is None and not f32:
        _check("zero_shard_step", load().zero_shard_step(*args, _stream_ptr(stream)))
    else:
        blocks, threads, path = launch if launch is not None else (0, 0, 0)
        opt = _Options(DTYPE_F32 if f32 else DTYPE_BF16, blocks, threads, path)
        _check("zero_shard_step_ex", load().zero_shard_step_ex(*args, C.byref(opt),
                                                                _stream_ptr(stream)))


def zero_shard_step_buckets(layout: Layout, hp: AdamW, t: int, bucket_begin: int,
                            bucket_end: int, rank_grads, grad_layout: int, master, exp_avg,
                            exp_avg_sq, param_out, out_mode: int, reduced_grad_out=None,
                            stream=None, launch=None):
    """The shard step of buckets [bucket_begin, bucket_end) only; the
    buffers are the whole-shard ones of zero_shard_step."""
    import torch
    if len(rank_grads) != layout.n_d:
        raise ValueError("zero_shard_step_buckets: one contribution per rank is required")
    f32 = len(rank_grads) > 0 and rank_grads[0] is not None and rank_grads[0].dtype == torch.float32
    blocks, threads, path = launch if launch is not None else (0, 0, 0)
    opt = _Options(DTYPE_F32 if f32 else DTYPE_BF16, blocks, threads, path)
    ng, ns, no = _step_sizes(layout, grad_layout, out_mode)
    _sizes((rank_grads, "rank_grads", ng), (master, "master", ns), (exp_avg, "exp_avg", ns),
           (exp_avg_sq, "exp_avg_sq", ns), (param_out, "param_out", no),
           (reduced_grad_out, "reduced_grad_out", ns))
    _check("zero_shard_step_buckets", load().zero_shard_step_buckets(
        layout.handle, C.byref(hp._c()), int(t), int(bucket_begin), int(bucket_end),
        _ptr_array(rank_grads, "rank_grads", _dev32 if f32 else _dev16, ng), grad_layout,
        _dev32(master, "master", ns), _dev32(exp_avg, "exp_avg", ns),
        _dev32(exp_avg_sq, "exp_avg_sq", ns), _dev16(param_out, "param_out", no), out_mode,
        _dev32(reduced_grad_out, "reduced_grad_out", ns), C.byref(opt), _stream_ptr(stream)))


def zero_shard_step_accumulate(layout: Layout, hp: AdamW, t: int, rank_acc, rank_micro,
                               micro_scale: float, contrib_dtype: int, grad_layout: int, master,
                               exp_avg, exp_avg_sq, param_out, out_mode: int,
                               reduced_grad_out=None, stream=None, launch=None):
    """One shard step whose contributions are the ranks' fp32 accumulators
    plus their scaled last micro-batch (rounded to bf16 for DTYPE_BF16)."""
    if len(rank_acc) != layout.n_d or len(rank_micro) != layout.n_d:
        raise ValueError("zero_shard_step_accumulate: one accumulator and one micro-batch "
                         "gradient per rank are required")
    blocks, threads, path = launch if launch is not None else (0, 0, 0)
    opt = _Options(contrib_dtype, blocks, threads, path)
    ng, ns, no = _step_sizes(layout, grad_layout, out_mode)
    _sizes((rank_acc, "rank_acc", ng), (rank_micro, "rank_micro", ng), (master, "master", ns),
           (exp_avg, "exp_avg", ns), (exp_avg_sq, "exp_avg_sq", ns),
           (param_out, "param_out", no), (reduced_grad_out, "reduced_grad_out", ns))
    _check("zero_shard_step_accumulate", load().zero_shard_step_accumulate(
        layout.handle, C.byref(hp._c()), int(t), _ptr_array(rank_acc, "rank_acc", _dev32, ng),
        _ptr_array(rank_micro, "rank_micro", n=ng), float(micro_scale), contrib_dtype,
        grad_layout, _dev32(master, "master", ns), _dev32(exp_avg, "exp_avg", ns),
        _dev32(exp_avg_sq, "exp_avg_sq", ns), _dev16(param_out, "param_out", no), out_mode,
        _dev32(reduced_grad_out, "reduced_grad_out", ns), C.byref(opt), _stream_ptr(stream)))


def zero_gather_params(layout: Layout, rank_shards, full_out, bucket_begin: int = 0,
                       bucket_end: int | None = None, stream=None):
    if len(rank_shards) != layout.n_d:
        raise ValueError("zero_gather_params: one shard per rank is required")
    end = layout.n_buckets if bucket_end is None else bucket_end
    _sizes((rank_shards, "rank_shards", layout.shard), (full_out, "full_out", layout.padded))
    _check("zero_gather_params", load().zero_gather_params(
        layout.handle, _ptr_array(rank_shards, "rank_shards", n=layout.shard), bucket_begin, end,
        _dev16(full_out, "full_out", layout.padded), _stream_ptr(stream)))


def zero_reshard(src: Layout, src_shards, dst: Layout, dst_shard, stream=None):
    """Re-cut one per-element array (float32 or 16-bit tensors) from src's
    shards to dst's shard."""
    import torch
    if len(src_shards) != src.n_d:
        raise ValueError("zero_reshard: one shard per source rank is required")
    _sizes((src_shards, "src_shards", src.shard), (dst_shard, "dst_shard", dst.shard))
    f32 = dst_shard.dtype == torch.float32
    chk = _dev32 if f32 else _dev16
    _check("zero_reshard", load().zero_reshard(
        src.handle, _ptr_array(src_shards, "src_shards", chk, src.shard), dst.handle,
        chk(dst_shard, "dst_shard", dst.shard), 4 if f32 else 2, _stream_ptr(stream)))


def zero_step_scalars(hp: AdamW, t: int):
    out = (C.c_float * 8)()
    _check("zero_step_scalars", load().zero_step_scalars(C.byref(hp._c()), t, out))
    return list(out)


def zero_placement_plan(nbytes, traffic, lane_bytes: int, n_lanes: int, align: int):
    """Byte offsets of the buffers inside one pool, and the pool size."""
    n = len(nbytes)
    if len(traffic) != n:
        raise ValueError("zero_placement_plan: one traffic figure per buffer is required")
    nb = (C.c_int64 * max(1, n))(*[int(x) for x in nbytes])
    tr = (C.c_double * max(1, n))(*[float(x) for x in traffic])
    offs = (C.c_int64 * max(1, n))()
    total = C.c_int64()
    _check("zero_placement_plan", load().zero_placement_plan(
        n, nb, tr, int(lane_bytes), int(n_lanes), int(align), offs, C.byref(total)))
    return [int(offs[k]) for k in range(n)], int(total.value)
