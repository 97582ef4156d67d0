"""Decode attention read directly from a low-rank-compressed KV cache, for
AMD Instinct MI355X (gfx950).

The computation lives in liblrkv.so (include/lrkv.h, HIP kernels under csrc/);
``binding`` is a ctypes layer with the same entry-point names, ``layout`` holds
host-side helpers for the buffer layouts.  Importing the package does not load
the library; the first call does, and raises if it is missing.
"""

from . import layout  # noqa: F401

__all__ = ["layout", "binding"]


def __getattr__(name):
    if name == "binding":
        import importlib
        return importlib.import_module(".binding", __name__)
    raise AttributeError(name)
