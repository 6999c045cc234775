"""Measurement helpers for bench.py: the same-mix streaming ceiling."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmeasure.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("measure/libmeasure.so is not built (run __graft_entry__.build())")
        lib = C.CDLL(_LIB_PATH)
        lib.stream_ceiling_launch.argtypes = [C.POINTER(C.c_void_p), C.c_int32,
                                              C.POINTER(C.c_void_p), C.c_void_p, C.c_int64,
                                              C.c_int32, C.c_int32, C.c_void_p]
        lib.stream_ceiling_launch.restype = C.c_int
        lib.stream_probe_launch.argtypes = [C.c_int32, C.POINTER(C.c_void_p), C.c_int32,
                                            C.POINTER(C.c_void_p), C.c_void_p, C.c_int64,
                                            C.c_int32, C.c_int32, C.c_void_p]
        lib.stream_probe_launch.restype = C.c_int
        _lib = lib
    return _lib


def stream_ceiling(grads, state, out, n: int, reps: int = 5):
    """Best bandwidth (GB/s of 2*N_d + 26 bytes per element) of the same-mix
    kernel over a few launch shapes and cache policies (non-temporal: none,
    contribution loads, contribution loads and stores, everything), on the
    given (scratch) buffers."""
    import torch
    lib = _load()
    nd = len(grads)
    g = (C.c_void_p * nd)(*[t.data_ptr() for t in grads])
    s = (C.c_void_p * 3)(*[t.data_ptr() for t in state])
    n = n // 512 * 512
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    best = (0.0, None)
    for bpc in (1, 2, 4):
        for pol in (0, 1, 5, 7):
            args = (g, nd, s, out.data_ptr(), n, cus * bpc, pol, stream.cuda_stream)
            if lib.stream_ceiling_launch(*args) != 0:
                raise RuntimeError("stream_ceiling_launch failed")
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                lib.stream_ceiling_launch(*args)
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            gbps = n * (2 * nd + 26) / (ms * 1e-3) / 1e9
            if gbps > best[0]:
                best = (gbps, {"blocks_per_cu": bpc, "nontemporal_policy": pol, "ms": ms})
    return best


def stream_probes(grads, state, out, n: int, reps: int = 5):
    """Pure-read and copy bandwidth (GB/s) on the given (scratch) buffers:
    the read of every byte the step reads (2*N_d + 12 per element), and a copy
    of state array 0 into state array 1 (8 bytes per element); best over a
    few launch shapes.  Overwrites state array 1 and `out`."""
    import torch
    lib = _load()
    nd = len(grads)
    g = (C.c_void_p * nd)(*[t.data_ptr() for t in grads])
    s = (C.c_void_p * 3)(*[t.data_ptr() for t in state])
    n = n // 512 * 512
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    res = {}
    for kind, name, bpe in ((0, "read", 2 * nd + 12), (1, "copy", 8)):
        best = (0.0, None)
        for bpc in (1, 2, 4, 8):
            for nt in (0, 1):
                args = (kind, g, nd, s, out.data_ptr(), n, cus * bpc, nt, stream.cuda_stream)
                if lib.stream_probe_launch(*args) != 0:
                    raise RuntimeError("stream_probe_launch failed")
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    lib.stream_probe_launch(*args)
                e1.record(stream)
                torch.cuda.synchronize()
                ms = e0.elapsed_time(e1) / reps
                gbps = n * bpe / (ms * 1e-3) / 1e9
                if gbps > best[0]:
                    best = (gbps, {"blocks_per_cu": bpc, "nontemporal": bool(nt), "ms": ms})
        res[name] = {"GBps": best[0], "config": best[1]}
    return res


def mix_ms(grads, state, out, n: int, reps: int = 4):
    """Milliseconds per launch of the same-mix kernel (every access
    non-temporal, one 256-thread block per CU, the step's chunk mapping) on
    the given buffers, after one untimed launch.  It moves the step's bytes
    in the step's pattern, so it ranks placements of the step's buffers as
    the step does (measured: the same best shift of the Llama-3-8B pool, and
    one within 0.04 % of the step's best for Llama-70B), while the step's own
    kernel stays out of the search."""
    import torch
    lib = _load()
    nd = len(grads)
    g = (C.c_void_p * nd)(*[t.data_ptr() for t in grads])
    s = (C.c_void_p * 3)(*[t.data_ptr() for t in state])
    n = n // 512 * 512
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    stream = torch.cuda.current_stream()
    args = (g, nd, s, out.data_ptr(), n, cus, 7, stream.cuda_stream)
    if lib.stream_ceiling_launch(*args) != 0:
        raise RuntimeError("stream_ceiling_launch failed")
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        lib.stream_ceiling_launch(*args)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps
