"""Builds the two libraries in-tree with hipcc for gfx950.

    python -m rank_kv_cache_lrkv_amd.build [-v]

Every HIP source under csrc/ is compiled to an object under _build/ (in
parallel) and linked into rank_kv_cache_lrkv_amd/liblrkv.so (include/lrkv.h);
the measurement kernels under probe/ go into liblrkv_probe.so
(include/lrkv_probe.h), which only the benchmark loads.  Packed float32 VALU
instructions are switched off for the device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
PROBE = os.path.join(PKG, "probe")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "liblrkv.so")
PROBE_LIB = os.path.join(PKG, "liblrkv_probe.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources(d=CSRC):
    return sorted(os.path.join(d, f) for f in os.listdir(d) if f.endswith(".hip"))


COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(os.path.dirname(src)) + "_" + os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, f"-I{INCLUDE}", f"-I{os.path.dirname(src)}", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if verbose and errs.strip():
        print(errs, flush=True)
    return obj


def _link(objs, lib: str, verbose: bool) -> str:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


def build(verbose: bool = False) -> str:
    """Compile every HIP source, link liblrkv.so and liblrkv_probe.so; returns
    the path of liblrkv.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs, psrcs = sources(CSRC), sources(PROBE)
    with ThreadPoolExecutor(max_workers=min(8, len(srcs) + len(psrcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs + psrcs))
    _link(objs[len(srcs):], PROBE_LIB, verbose)
    return _link(objs[:len(srcs)], LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
