"""Seeded synthetic inputs, shared by the tests, the smoke check and the
benchmark.  Input recipe only: no step of the update happens here.

A value is a function of (stream key, global parameter index) alone, so the
GPU can fill hundreds of GB of rank contributions while the CPU regenerates
any sampled element for the oracle.  See synth_gen.hip for the generator and
the distributions.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

from . import workloads  # noqa: F401

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

DISTS = {"zero": 0, "normal": 1, "absnormal": 2, "student_t3": 3, "normal_zeros": 4}
OUT_F32, OUT_BF16 = 0, 1
KIND = {"grad": 1, "master": 2, "exp_avg": 3, "exp_avg_sq": 4, "micro_grad": 5}
WORKLOAD_ID = {name: k + 1 for k, name in enumerate(workloads.NAMES + workloads.DIM0_NAMES)}
# the padded-tail cut of the 70B list draws the same values as the plain cut
WORKLOAD_ID["llama70b_t"] = WORKLOAD_ID["llama70b"]
HOST_THREADS = max(1, min(16, os.cpu_count() or 1))


class Seg(C.Structure):
    _fields_ = [("dst_off", C.c_int64), ("x0", C.c_int64), ("n_real", C.c_int64),
                ("n_pad", C.c_int64)]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError("synth/libsynth.so is not built (run __graft_entry__.build())")
    lib = C.CDLL(_LIB_PATH)
    lib.synth_key.argtypes = [C.c_uint32] * 5
    lib.synth_key.restype = C.c_uint64
    lib.synth_philox.argtypes = [C.POINTER(C.c_uint32)] * 3
    lib.synth_fill_host.argtypes = [C.c_void_p, C.c_int32, C.POINTER(Seg), C.c_int32, C.c_uint64,
                                    C.c_int32, C.c_double, C.c_int32]
    lib.synth_values_at.argtypes = [C.POINTER(C.c_int64), C.c_int64, C.c_uint64, C.c_int32,
                                    C.c_double, C.c_int32, C.c_void_p, C.c_int32]
    lib.synth_fill_device.argtypes = [C.c_void_p, C.c_int64, C.c_int32, C.POINTER(Seg), C.c_int32,
                                      C.c_uint64, C.c_int32, C.c_double, C.c_void_p]
    for f in (lib.synth_fill_host, lib.synth_values_at, lib.synth_fill_device):
        f.restype = C.c_int
    _lib = lib
    return lib


def key(workload: str, kind: str, rank: int = 0, micro: int = 0, step: int = 0) -> int:
    return _load().synth_key(WORKLOAD_ID[workload], KIND[kind], rank, micro, step)


def philox(ctr, k):
    c = (C.c_uint32 * 4)(*ctr)
    kk = (C.c_uint32 * 2)(*k)
    out = (C.c_uint32 * 4)()
    _load().synth_philox(c, kk, out)
    return list(out)


def _segs(segs):
    arr = (Seg * max(1, len(segs)))()
    for i, s in enumerate(segs):
        arr[i] = Seg(*[int(v) for v in s])
    return arr


def _np_dtype(out_type):
    return np.float32 if out_type == OUT_F32 else np.uint16


def fill_host(n_out: int, out_type: int, segs, key_: int, dist: str, scale: float,
              nthreads: int = HOST_THREADS) -> np.ndarray:
    out = np.zeros(n_out, _np_dtype(out_type))
    rc = _load().synth_fill_host(out.ctypes.data, out_type, _segs(segs), len(segs), key_,
                                 DISTS[dist], scale, nthreads)
    if rc:
        raise ValueError(f"synth_fill_host rc={rc}")
    return out


def values_at(xs, key_: int, dist: str, scale: float, out_type: int,
              nthreads: int = HOST_THREADS) -> np.ndarray:
    xs = np.ascontiguousarray(xs, dtype=np.int64)
    out = np.empty(xs.size, _np_dtype(out_type))
    rc = _load().synth_values_at(xs.ctypes.data_as(C.POINTER(C.c_int64)), xs.size, key_,
                                 DISTS[dist], scale, out_type, out.ctypes.data, nthreads)
    if rc:
        raise ValueError(f"synth_values_at rc={rc}")
    return out


def fill_device(tensor, segs, key_: int, dist: str, scale: float, stream=None) -> None:
    """Fill a contiguous torch CUDA tensor (float32, or a 16-bit dtype holding
    bf16 bits) over `segs` on the current (or given) stream."""
    import torch
    assert tensor.is_cuda and tensor.is_contiguous()
    out_type = OUT_F32 if tensor.dtype == torch.float32 else OUT_BF16
    if out_type == OUT_BF16:
        assert tensor.element_size() == 2
    s = stream if stream is not None else torch.cuda.current_stream()
    rc = _load().synth_fill_device(tensor.data_ptr(), tensor.numel(), out_type, _segs(segs),
                                   len(segs), key_, DISTS[dist], scale, s.cuda_stream)
    if rc:
        raise ValueError(f"synth_fill_device rc={rc}")


# ------------------------------------------------------------ segment builders
def shard_segments(stream_off, length, padded_len, shard_off, n_d: int, rank: int):
    """Segments that lay out rank `rank`'s shard (its slice of every padded
    bucket, in bucket order) with values keyed by the global parameter index;
    bucket padding becomes zeros."""
    segs = []
    for so, ln, pl, sh in zip(stream_off, length, padded_len, shard_off):
        sb = int(pl) // n_d
        n_real = max(0, min(sb, int(ln) - rank * sb))
        segs.append((int(sh), int(so) + rank * sb, n_real, sb - n_real))
    return segs


def tensor_segments(numel):
    """One segment per tensor, each starting at offset 0 of its own buffer."""
    out, off = [], 0
    for n in numel:
        out.append([(0, off, int(n), 0)])
        off += int(n)
    return out
