"""ctypes binding of liblrkv_probe.so (include/lrkv_probe.h): the measurement
kernels the benchmark uses beside the library -- a plain HBM read stream (the
bandwidth ceiling for reading the decode's bytes) and a bounded spin that keeps
the GPU busy while a host loop enqueues the launches it times.  Argument
marshalling only; loading raises if the library is missing."""

from __future__ import annotations

import ctypes
import os
import threading
from ctypes import c_int32, c_int64, c_void_p

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblrkv_probe.so")

SIGNATURES = [
    ("lrkv_probe_read", c_int32, [c_void_p, c_int64, c_void_p, c_int32, c_int32, c_int32, c_void_p]),
    ("lrkv_probe_spin", c_int32, [c_int64, c_void_p, c_void_p]),
    ("lrkv_probe_wall_clock_khz", c_int32, []),
]

_lib = None
_lock = threading.Lock()


def lib():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing: build the libraries first "
                                   "(python -m rank_kv_cache_lrkv_amd.build)")
            h = ctypes.CDLL(LIB_PATH)
            for name, res, args in SIGNATURES:
                f = getattr(h, name)
                f.restype = res
                f.argtypes = args
            _lib = h
    return _lib


def _check(st, where):
    if st != 0:
        raise RuntimeError(f"{where}: status {st}")


def read(src, nbytes: int, sink, grid: int, unroll: int, nontemporal: bool, stream: int):
    """One read-stream launch over the first ``nbytes`` bytes of device tensor ``src``."""
    _check(lib().lrkv_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), grid, unroll, int(nontemporal),
                                 stream), "lrkv_probe_read")


def spin_us(us: float, sink, stream: int):
    """Keep the GPU busy for about ``us`` microseconds (bounded wait)."""
    khz = lib().lrkv_probe_wall_clock_khz()
    if khz <= 0:
        raise RuntimeError("wall clock rate unavailable")
    ticks = int(min(us * khz / 1000.0, float(1 << 32)))
    _check(lib().lrkv_probe_spin(ticks, sink.data_ptr(), stream), "lrkv_probe_spin")


def exported_names():
    return [s[0] for s in SIGNATURES]
