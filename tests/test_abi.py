"""The C-ABI library on the CPU: it loads, exports every entry point that
include/lrkv.h declares, and rejects bad arguments on the host before any HIP
call (no compute is launched here)."""

import ctypes
import os
import re

import numpy as np
import pytest

from rank_kv_cache_lrkv_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "lrkv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lrkv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_binding_entry_points():
    assert declared_functions() == sorted(B.exported_names())


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    out = os.popen(f"nm -D --defined-only {B.LIB_PATH}").read()
    for name in declared_functions():
        assert re.search(rf"\bT {name}\b", out), name


def test_status_strings_and_version():
    lib = B.lib()
    assert lib.lrkv_status_string(0) == b"ok"
    for s in range(1, 9):
        assert lib.lrkv_status_string(s) not in (b"ok", b"unknown status")
    assert lib.lrkv_version() >= 100


FAKE = 1 << 20   # a 16-byte-aligned non-null address; validation fails before any use


def layer(**kw):
    d = dict(dtype=1, batch=2, n_q_heads=8, n_kv_heads=2, window=4, cap=64,
             rank_k=[64, 32], rank_v=[32, 16])
    d.update(kw)
    rk = (ctypes.c_int32 * len(d["rank_k"]))(*d["rank_k"])
    rv = (ctypes.c_int32 * len(d["rank_v"]))(*d["rank_v"])
    s = B.lrkv_layer(d["dtype"], d["batch"], d["n_q_heads"], d["n_kv_heads"], d["window"], d["cap"],
                     ctypes.cast(rk, ctypes.POINTER(ctypes.c_int32)),
                     ctypes.cast(rv, ctypes.POINTER(ctypes.c_int32)),
                     d.get("bases", FAKE), d.get("codes_k", FAKE), d.get("codes_v", FAKE),
                     d.get("anchor_k", FAKE), d.get("anchor_v", FAKE),
                     d.get("scales_k", FAKE), d.get("scales_v", FAKE))
    s._keep = (rk, rv)
    return s


def decode(L, n_ctx=50, q=FAKE, out=FAKE, scale=0.088, S=2, ws=FAKE, ws_bytes=1 << 30):
    return B.lib().lrkv_decode_attn(ctypes.byref(L), n_ctx, None, q, out, scale, S, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), 4),
    (dict(batch=0), 2),
    (dict(batch=32768), 2),                                     # 65536 (row, head) units
    (dict(n_q_heads=7), 2),
    (dict(n_q_heads=2 * 17, n_kv_heads=2), 2),
    (dict(window=-1), 2),
    (dict(cap=40), 2),
    (dict(cap=(1 << 31) // 256 // 32 * 32 + 32), 2),          # bf16 code region past 2^31 bytes
    (dict(dtype=0, cap=(1 << 31) // 512 // 32 * 32 + 32), 2),
    (dict(rank_k=[64, 24]), 3),
    (dict(rank_v=[32, 0]), 3),
    (dict(rank_k=[144, 32]), 3),
    (dict(bases=None), 1),
    (dict(codes_v=None), 1),
    (dict(anchor_k=FAKE + 8), 5),
    (dict(dtype=2, scales_k=None), 1),                          # int8 codes need their scales
    (dict(dtype=2, scales_v=FAKE + 4), 5),
    (dict(dtype=2, cap=(1 << 31) // 256 // 32 * 32 + 32), 2),
    (dict(dtype=3, scales_v=None), 1),                          # 4-bit codes too
    (dict(dtype=4), 4),
])
def test_layer_validation(kw, status):
    assert decode(layer(**kw)) == status


def test_decode_argument_validation():
    L = layer()
    assert decode(L, n_ctx=0) == 2
    assert decode(L, n_ctx=4 + 64 + 2) == 6           # needs 65 code slots, cap is 64
    assert decode(L, q=None) == 1
    assert decode(L, out=None) == 1
    assert decode(L, out=FAKE + 4) == 5
    assert decode(L, S=-1) == 2
    assert decode(L, S=B.lib().lrkv_decode_workspace_size(ctypes.byref(L), 1) and 1025) == 2
    assert decode(L, scale=0.0) == 2
    assert decode(L, scale=float("nan")) == 2
    assert decode(L, ws=None) == 7
    need = B.lib().lrkv_decode_workspace_size(ctypes.byref(L), 2)
    assert decode(L, ws_bytes=need - 1) == 7


def test_workspace_size_formula():
    L = layer()
    lib = B.lib()
    # one record of 4 + max r_v (32) + 128 floats per (row, query head, split)
    assert lib.lrkv_decode_workspace_size(ctypes.byref(L), 3) == 2 * 8 * 3 * (4 + 32 + 128) * 4
    assert lib.lrkv_decode_workspace_size(ctypes.byref(L), 0) == 0
    assert lib.lrkv_decode_workspace_size(ctypes.byref(layer(batch=0)), 3) == 0


def test_auto_splits():
    lib = B.lib()
    # Llama-3.1-8B-shaped layer at 32K: 32 (row, KV head) units -> 32 splits
    L = layer(batch=4, n_q_heads=32, n_kv_heads=8, window=128, cap=32768,
              rank_k=[64] * 8, rank_v=[32] * 8)
    assert lib.lrkv_decode_auto_splits(ctypes.byref(L), 32768) == 32
    assert lib.lrkv_decode_auto_splits(ctypes.byref(L), 100) == 1
    assert lib.lrkv_decode_auto_splits(ctypes.byref(L), 0) == 0
    # Qwen3-1.7B-shaped layer at 4K: 64 units could take 16 splits each, but a split
    # keeps at least 16 of the row's 126 code blocks (4 per wave): 8 splits
    Lq = layer(batch=8, n_q_heads=16, n_kv_heads=8, window=64, cap=4096, rank_k=[64] * 8, rank_v=[32] * 8)
    assert lib.lrkv_decode_auto_splits(ctypes.byref(Lq), 4096) == 8
    # float32 storage keeps at least 4 blocks a split
    Lf = layer(dtype=0, batch=1, n_q_heads=1, n_kv_heads=1, window=16, cap=256, rank_k=[64], rank_v=[32])
    assert lib.lrkv_decode_auto_splits(ctypes.byref(Lf), 256) == 2
    # the pre-RoPE and LowRAM kernels fit three workgroups per compute unit: 768 / 32 = 24
    L.rope_base = 500000.0
    assert lib.lrkv_decode_auto_splits(ctypes.byref(L), 32768) == 24


def test_compress_validation():
    lib = B.lib()
    L = layer()
    f = lambda **k: lib.lrkv_compress(ctypes.byref(L), k.get("which", 0), k.get("x", FAKE),
                                      k.get("sb", 1024), k.get("sh", 512), k.get("st", 128),
                                      k.get("n", 10), k.get("slot0", 0), None)
    assert f(which=2) == 2
    assert f(n=-1) == 2
    assert f(slot0=-1) == 2
    assert f(n=60, slot0=5) == 6
    assert f(n=0, x=None) == 0           # empty range is a no-op
    assert f(x=None) == 1
    assert f(st=100) == 5                 # 200-byte row stride is not 16-byte aligned
    assert f(sh=-512) == 2
    assert f(x=FAKE + 2) == 5


def test_store_and_append_validation():
    lib = B.lib()
    L = layer()
    sa = lambda pos0, n, k=FAKE: lib.lrkv_store_anchors(ctypes.byref(L), k, FAKE, 1024, 512, 128, pos0, n, None)
    assert sa(0, 6) == 2          # 1 + window = 5 slots
    assert sa(3, 5) == 2          # 4 ring slots
    assert sa(-1, 1) == 2
    assert sa(0, 0) == 0
    assert sa(0, 2, k=None) == 1
    ap = lambda pos, k=FAKE: lib.lrkv_append(ctypes.byref(L), k, FAKE, pos, None)
    assert ap(-1) == 2
    assert ap(4 + 64 + 1) == 6    # would compress into slot 64 of a 64-slot region
    assert ap(5, k=None) == 1
    assert ap(5, k=FAKE + 2) == 5
    L0 = layer(window=0)
    assert lib.lrkv_store_anchors(ctypes.byref(L0), FAKE, FAKE, 1024, 512, 128, 1, 1, None) == 2
    assert lib.lrkv_append(ctypes.byref(L0), FAKE, FAKE, 65, None) == 6


def test_scales_ignored_unless_int8():
    # bf16 and f32 layers never read the scale pointers: null is fine
    L = layer(scales_k=None, scales_v=None)
    assert decode(L, q=None) == 1     # fails on q, not on the scales
    L8 = layer(dtype=2)
    assert decode(L8, q=None) == 1


def test_quantize_validation():
    lib = B.lib()
    L8 = layer(dtype=2)
    f = lambda L=L8, **k: lib.lrkv_quantize(ctypes.byref(L), k.get("which", 0), k.get("x", FAKE),
                                           k.get("sb", 1024), k.get("sh", 512), k.get("st", 65),
                                           k.get("n", 10), k.get("slot0", 0), None)
    assert f(L=layer(dtype=1)) == 4      # only int8-code layers
    assert f(L=layer(dtype=0)) == 4
    assert f(which=2) == 2
    assert f(n=-1) == 2
    assert f(slot0=-1) == 2
    assert f(n=60, slot0=5) == 6
    assert f(n=0, x=None) == 0           # empty range is a no-op
    assert f(x=None) == 1
    assert f(sh=-512) == 2
    assert f(x=FAKE + 2) == 5            # float32 rows need 4-byte alignment only
    assert f(L=layer(dtype=2, scales_v=None)) == 1
    assert f(L=layer(dtype=3), n=60, slot0=5) == 6     # 4-bit layers take the same checks
    assert f(L=layer(dtype=3), x=FAKE + 2) == 5


def test_versions_validation():
    # 0 versions is read as 1; more than LRKV_MAX_VERSIONS (16) or a missing or
    # misaligned start table is rejected
    assert decode(layer(n_versions=0), q=None) == 1
    L = layer()
    L.n_versions = 17
    assert decode(L) == 2
    L.n_versions = 2
    assert decode(L) == 1                   # version_start missing
    L.version_start = FAKE + 2
    assert decode(L) == 5


def test_oja_validation():
    lib = B.lib()
    L = layer()
    need = lib.lrkv_oja_workspace_size(ctypes.byref(L))
    assert need == 2 * (64 * 36 * 256 + 128 * 128) * 4  # 2 KV heads x (64 workgroup partials of 36 tiles + C in full)
    f = lambda L=L, **k: lib.lrkv_oja_update(ctypes.byref(L), k.get("which", 0), k.get("x", FAKE), 1024, 512,
                                             128, k.get("n", 10), k.get("eta", 0.5), k.get("vin", 0),
                                             k.get("vout", 0), k.get("ws", FAKE), k.get("wsb", need), None)
    assert f(L=layer(dtype=0)) == 4
    assert f(which=2) == 2
    assert f(n=0) == 2
    assert f(eta=float("nan")) == 2
    assert f(vout=1) == 2                    # one version only
    assert f(x=None) == 1
    assert f(x=FAKE + 2) == 5
    assert f(wsb=need - 1) == 7
    assert f(ws=None) == 7


def test_head_group_validation():
    def grouped(hg, **kw):
        L = layer(**kw)
        L.head_group = hg
        return L
    one = dict(rank_k=[64], rank_v=[32])    # one latent group of both KV heads
    assert decode(grouped(2, **one), q=None) == 1      # a valid layer: fails on q only
    assert decode(grouped(0), q=None) == 1             # 0 and 1: one code stream per KV head
    assert decode(grouped(1), q=None) == 1
    assert decode(grouped(3, **one)) == 2              # 2 KV heads are not groups of 3
    assert decode(grouped(16, n_kv_heads=16, n_q_heads=16, rank_k=[64], rank_v=[32])) == 2  # > 8
    assert decode(grouped(2, n_q_heads=2 * 16, **one)) == 2   # 2 x 16 query heads per group > 16
    assert decode(grouped(2, dtype=0, **one)) == 4     # float32 storage has no groups
    assert decode(grouped(2, rank_k=[64], rank_v=[24])) == 3
    lib = B.lib()
    L = grouped(2, **one)
    # the auto split count depends on the code streams (one here), not the KV heads
    assert lib.lrkv_decode_auto_splits(ctypes.byref(L), 32768) >= \
        lib.lrkv_decode_auto_splits(ctypes.byref(layer()), 32768)
    assert lib.lrkv_oja_update(ctypes.byref(L), 0, FAKE, 1024, 512, 128, 10, 0.5, 0, 0, FAKE, 1 << 30,
                               None) == 2      # the Oja step is per KV head


def test_lowram_validation():
    def lowram(r=4, **kw):
        L = layer(**kw)
        L.value_mode, L.resid_per_block = 1, r
        L.predictor, L.resid, L.resid_slot, L.resid_norm = FAKE, FAKE, FAKE, FAKE
        return L
    assert decode(lowram(), q=None) == 1                # a valid layer: fails on q only
    assert decode(lowram(codes_v=None), q=None) == 1    # no value codes needed
    assert decode(layer(codes_v=None)) == 1               # value codes needed otherwise
    bad = layer()
    bad.value_mode = 2
    assert decode(bad) == 4
    assert decode(lowram(r=0)) == 2
    assert decode(lowram(r=9)) == 2                     # > LRKV_MAX_RESID
    assert decode(lowram(dtype=2)) == 4                 # bf16 codes only
    L = lowram()
    L.head_group = 2
    assert decode(L) == 4
    L = lowram()
    L.predictor = None
    assert decode(L) == 1
    L = lowram()
    L.resid = FAKE + 8
    assert decode(L) == 5
    lib = B.lib()
    L = lowram()
    need = lib.lrkv_lowram_workspace_size(ctypes.byref(L))
    assert need == 4 * 16 * 64 * (64 + 128) * 4      # 4 units x 16 partials x r x (r + 128) floats
    assert lib.lrkv_lowram_workspace_size(ctypes.byref(layer())) == 0
    fit = lambda L=L, **k: lib.lrkv_lowram_fit(ctypes.byref(L), k.get("v", FAKE), 1024, 512, 128, k.get("n", 10),
                                               k.get("ws", FAKE), k.get("wsb", need), None)
    assert fit(L=layer()) == 4
    assert fit(n=0) == 2
    assert fit(n=65) == 6                                # cap 64
    assert fit(v=None) == 1
    assert fit(v=FAKE + 2) == 5
    assert fit(wsb=need - 1) == 7
    assert lib.lrkv_compress(ctypes.byref(L), 1, FAKE, 1024, 512, 128, 10, 0, None) == 4


def test_rope_validation():
    def roped(base, **kw):
        L = layer(**kw)
        L.rope_base = base
        return L
    assert decode(roped(10000.0), q=None) == 1          # a valid layer: fails on q only
    assert decode(roped(0.5)) == 2
    assert decode(roped(float("inf"))) == 2
    assert decode(roped(float("nan"))) == 2
    assert decode(roped(10000.0, dtype=2)) == 4          # bf16 codes only
    L = roped(10000.0)
    L.head_group = 2
    L.rank_k = L.rank_k                                  # (one rank per KV head stays valid)
    assert decode(L) in (2, 4)
    L = roped(10000.0)
    L.n_versions, L.version_start = 2, FAKE
    assert decode(L) == 4
    L = roped(10000.0)
    L.value_mode, L.resid_per_block = 1, 4
    L.predictor, L.resid, L.resid_slot, L.resid_norm = FAKE, FAKE, FAKE, FAKE
    assert decode(L) == 4


PROBE_HEADER = os.path.join(os.path.dirname(HEADER), "lrkv_probe.h")


def test_probe_library_exports_its_header():
    """The measurement library (read stream, spin) exports what lrkv_probe.h
    declares, and the binding names the same functions."""
    from rank_kv_cache_lrkv_amd import measure
    text = re.sub(r"/\*.*?\*/", "", open(PROBE_HEADER).read(), flags=re.S)
    declared = sorted(set(re.findall(r"\b(lrkv_probe_[a-z_]+)\s*\(", text)))
    assert declared == sorted(measure.exported_names())
    lib = measure.lib()
    out = os.popen(f"nm -D --defined-only {measure.LIB_PATH}").read()
    for name in declared:
        assert hasattr(lib, name), name
        assert re.search(rf"\bT {name}\b", out), name


@pytest.mark.parametrize("args,status", [
    ((None, 1 << 20, FAKE, 1024, 4, 0), 1),     # null source
    ((FAKE, 1 << 20, None, 1024, 4, 0), 1),     # null sink
    ((FAKE, 0, FAKE, 1024, 4, 0), 2),           # no bytes
    ((FAKE, 1000, FAKE, 1024, 4, 0), 2),        # not a multiple of 16
    ((FAKE, 1 << 20, FAKE, 0, 4, 0), 2),        # empty grid
    ((FAKE, 1 << 20, FAKE, 70000, 4, 0), 2),    # grid past 65535
    ((FAKE, 1 << 20, FAKE, 1024, 3, 0), 2),     # unroll not 1, 2, 4 or 8
    ((FAKE + 8, 1 << 20, FAKE, 1024, 4, 0), 5), # misaligned source
])
def test_probe_read_rejects_bad_arguments(args, status):
    from rank_kv_cache_lrkv_amd import measure
    assert measure.lib().lrkv_probe_read(*args, None) == status


def test_probe_spin_rejects_bad_arguments():
    from rank_kv_cache_lrkv_amd import measure
    assert measure.lib().lrkv_probe_spin(100, None, None) == 1
    assert measure.lib().lrkv_probe_spin(-1, FAKE, None) == 2
    assert measure.lib().lrkv_probe_spin((1 << 32) + 1, FAKE, None) == 2


def test_noalloc_decode_validates_on_the_host():
    """lrkv_decode_attn_noalloc checks every argument before any HIP call, and
    rejects split records larger than its 16 MiB array."""
    lib = B.lib()
    L = layer(batch=64, n_q_heads=32, n_kv_heads=8, window=32, cap=96, rank_k=[32] * 8, rank_v=[32] * 8)
    f = lambda **k: lib.lrkv_decode_attn_noalloc(ctypes.byref(L), k.get("n", 100), None, k.get("q", FAKE),
                                                 k.get("out", FAKE), 0.088, k.get("S", 2), None)
    assert f(q=None) == 1
    assert f(out=FAKE + 4) == 5
    assert f(n=0) == 2
    assert f(n=10000) == 6
    assert lib.lrkv_decode_workspace_size(ctypes.byref(L), 1024) > B.NOALLOC_CAPACITY
    assert f(S=1024) == 7
