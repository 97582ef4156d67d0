"""Thin ctypes binding of liblrkv.so (include/lrkv.h).

Argument marshalling only: torch supplies device memory and the current HIP
stream; every step of the computation runs in the library's kernels.  The
functions keep the C names.  There is no fallback: if the library is missing
and cannot be built, loading raises.
"""

from __future__ import annotations

import ctypes
import os
import threading
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

from . import layout

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblrkv.so")

LRKV_F32, LRKV_BF16, LRKV_BF16_Q8, LRKV_BF16_Q4 = 0, 1, 2, 3
QUANTISED = (LRKV_BF16_Q8, LRKV_BF16_Q4)
LRKV_VALUES_CODES, LRKV_VALUES_LOWRAM = 0, 1
HEAD_DIM = 128
BLOCK = 32

STATUS = {
    0: "LRKV_OK", 1: "LRKV_ERR_NULL", 2: "LRKV_ERR_SHAPE", 3: "LRKV_ERR_RANK",
    4: "LRKV_ERR_DTYPE", 5: "LRKV_ERR_ALIGN", 6: "LRKV_ERR_CAPACITY",
    7: "LRKV_ERR_WORKSPACE", 8: "LRKV_ERR_HIP",
}


class LrkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({_status_string(status)})")


class lrkv_layer(ctypes.Structure):
    _fields_ = [
        ("dtype", c_int32), ("batch", c_int32), ("n_q_heads", c_int32),
        ("n_kv_heads", c_int32), ("window", c_int32), ("cap", c_int32),
        ("rank_k", POINTER(c_int32)), ("rank_v", POINTER(c_int32)),
        ("bases", c_void_p), ("codes_k", c_void_p), ("codes_v", c_void_p),
        ("anchor_k", c_void_p), ("anchor_v", c_void_p),
        ("scales_k", c_void_p), ("scales_v", c_void_p),
        ("n_versions", c_int32), ("version_start", c_void_p),
        ("head_group", c_int32),
        ("value_mode", c_int32), ("resid_per_block", c_int32),
        ("predictor", c_void_p), ("resid", c_void_p), ("resid_slot", c_void_p), ("resid_norm", c_void_p),
        ("rope_base", c_float),
    ]


_lib = None
_lock = threading.Lock()

# (name, restype, argtypes) for every entry point of include/lrkv.h
_P = POINTER(lrkv_layer)
SIGNATURES = [
    ("lrkv_compress", c_int32, [_P, c_int32, c_void_p, c_int64, c_int64, c_int64, c_int32, c_int32, c_void_p]),
    ("lrkv_quantize", c_int32, [_P, c_int32, c_void_p, c_int64, c_int64, c_int64, c_int32, c_int32, c_void_p]),
    ("lrkv_lowram_workspace_size", c_size_t, [_P]),
    ("lrkv_lowram_fit", c_int32, [_P, c_void_p, c_int64, c_int64, c_int64, c_int32, c_void_p, c_size_t,
                                  c_void_p]),
    ("lrkv_oja_workspace_size", c_size_t, [_P]),
    ("lrkv_oja_update", c_int32, [_P, c_int32, c_void_p, c_int64, c_int64, c_int64, c_int32, c_float,
                                  c_int32, c_int32, c_void_p, c_size_t, c_void_p]),
    ("lrkv_store_anchors", c_int32, [_P, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_int32, c_int32, c_void_p]),
    ("lrkv_append", c_int32, [_P, c_void_p, c_void_p, c_int32, c_void_p]),
    ("lrkv_decode_workspace_size", c_size_t, [_P, c_int32]),
    ("lrkv_decode_auto_splits", c_int32, [_P, c_int32]),
    ("lrkv_decode_partials", c_int32, [_P, c_int32, c_void_p, c_void_p, c_float, c_int32, c_void_p, c_size_t, c_void_p]),
    ("lrkv_decode_combine", c_int32, [_P, c_int32, c_void_p, c_int32, c_void_p, c_size_t, c_void_p,
                                      c_void_p]),
    ("lrkv_decode_attn", c_int32, [_P, c_int32, c_void_p, c_void_p, c_void_p, c_float, c_int32, c_void_p, c_size_t, c_void_p]),
    ("lrkv_decode_attn_noalloc", c_int32, [_P, c_int32, c_void_p, c_void_p, c_void_p, c_float, c_int32,
                                           c_void_p]),
    ("lrkv_status_string", ctypes.c_char_p, [c_int32]),
    ("lrkv_version", c_int32, []),
]


def lib():
    """Load liblrkv.so (building it first only if it does not exist)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                from .build import build
                build()
            h = ctypes.CDLL(LIB_PATH)
            for name, res, args in SIGNATURES:
                f = getattr(h, name)
                f.restype = res
                f.argtypes = args
            _lib = h
    return _lib


def _status_string(status: int) -> str:
    try:
        return lib().lrkv_status_string(status).decode()
    except Exception:  # pragma: no cover - only while reporting another error
        return "?"


def _check(status: int, where: str):
    if status != 0:
        raise LrkvError(status, where)


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


# ---------------------------------------------------------------------------
# a layer of compressed cache in torch-owned device memory
# ---------------------------------------------------------------------------

@dataclass
class Layer:
    """One layer of compressed cache.  The tensors follow the layouts of lrkv.h;
    ``struct`` is the C description handed to every call."""

    dtype: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    window: int
    cap: int
    rank_k: np.ndarray
    rank_v: np.ndarray
    bases: "object"
    codes_k: "object"
    codes_v: "object"
    anchor_k: "object"
    anchor_v: "object"
    scales_k: "object" = None  # quantised codes only: float32 [n_latent][batch][cap]
    scales_v: "object" = None
    n_versions: int = 1
    version_start: "object" = None  # int32 [batch][n_versions] (device) when n_versions > 1
    head_group: int = 1  # KV heads sharing one code stream; rank_k / rank_v per group
    value_mode: int = LRKV_VALUES_CODES
    resid_per_block: int = 0  # LowRAM: residual entries per 32-slot block
    predictor: "object" = None  # LowRAM: bf16 M(b, h) rows
    resid: "object" = None      # LowRAM: bf16 [n_kv][batch][cap / 32][R][128]
    resid_slot: "object" = None  # LowRAM: int32 [n_kv][batch][cap / 32][R]
    resid_norm: "object" = None  # LowRAM: float32, same shape
    rope_base: float = 0.0  # > 1: key codes are of pre-RoPE keys (rotate-half RoPE with this base)
    _rk: object = field(default=None, repr=False)
    _rv: object = field(default=None, repr=False)
    struct: lrkv_layer = field(default=None, repr=False)

    def __post_init__(self):
        self._rk = (c_int32 * max(1, len(self.rank_k)))(*[int(x) for x in self.rank_k])
        self._rv = (c_int32 * max(1, len(self.rank_v)))(*[int(x) for x in self.rank_v])
        self.struct = lrkv_layer(
            self.dtype, self.batch, self.n_q_heads, self.n_kv_heads, self.window, self.cap,
            ctypes.cast(self._rk, POINTER(c_int32)), ctypes.cast(self._rv, POINTER(c_int32)),
            _ptr(self.bases), _ptr(self.codes_k), _ptr(self.codes_v),
            _ptr(self.anchor_k), _ptr(self.anchor_v), _ptr(self.scales_k), _ptr(self.scales_v),
            int(self.n_versions), _ptr(self.version_start), int(self.head_group),
            int(self.value_mode), int(self.resid_per_block), _ptr(self.predictor), _ptr(self.resid),
            _ptr(self.resid_slot), _ptr(self.resid_norm), float(self.rope_base))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_latent(self) -> int:
        """Code streams per batch row: KV heads, or head groups."""
        return self.n_kv_heads // max(1, self.head_group)

    @property
    def torch_dtype(self):
        """Storage type of bases, anchors, queries and compress inputs."""
        import torch
        return torch.float32 if self.dtype == LRKV_F32 else torch.bfloat16

    @property
    def code_dtype(self):
        """Element type of the codes tensors (4-bit codes: uint8 bytes, two per byte)."""
        import torch
        if self.dtype == LRKV_BF16_Q4:
            return torch.uint8
        return torch.int8 if self.dtype == LRKV_BF16_Q8 else self.torch_dtype

    @classmethod
    def allocate(cls, *, dtype: int, batch: int, n_q_heads: int, n_kv_heads: int, window: int,
                 cap: int, rank_k: Sequence[int], rank_v: Sequence[int], device="cuda",
                 bases=None, n_versions: int = 1, head_group: int = 1, lowram_resid: int = 0,
                 rope_base: float = 0.0) -> "Layer":
        """Allocate zeroed codes and anchors (and int8 scales) (torch) for the given
        geometry.  ``bases`` (optional) is the flat bases tensor; otherwise zeros.
        With ``head_group`` > 1, rank_k / rank_v hold one rank per group of
        ``head_group`` KV heads.  ``lowram_resid`` = R > 0 makes a LowRAM layer
        (values predicted from the key codes, R residual rows per block): no value
        codes, a zeroed predictor and empty residual entries."""
        import torch
        td = torch.float32 if dtype == LRKV_F32 else torch.bfloat16
        cd = {LRKV_BF16_Q8: torch.int8, LRKV_BF16_Q4: torch.uint8}.get(dtype, td)
        per = 2 if dtype == LRKV_BF16_Q4 else 1  # code elements per tensor element
        rk = np.asarray(rank_k, np.int32)
        rv = np.asarray(rank_v, np.int32)
        cap = layout.round_cap(cap)
        hg = max(1, int(head_group))
        n_lat = n_kv_heads // hg
        nb = layout.bases_elems(rk, rv, hg) * n_versions   # one copy of the layout per version
        if bases is None:
            bases = torch.zeros(nb, dtype=td, device=device)
        assert bases.numel() == nb and bases.dtype == td
        ck = torch.zeros(max(1, layout.codes_elems(rk, batch, cap) // per), dtype=cd, device=device)
        cv = torch.zeros(max(1, layout.codes_elems(rv, batch, cap) // per), dtype=cd, device=device)
        ak = torch.zeros((batch, n_kv_heads, 1 + window, HEAD_DIM), dtype=td, device=device)
        av = torch.zeros_like(ak)
        sk = sv = None
        if dtype in QUANTISED:
            sk = torch.zeros(max(1, layout.scales_elems(n_lat, batch, cap)), dtype=torch.float32,
                             device=device)
            sv = torch.zeros_like(sk)
        vs = torch.zeros((batch, n_versions), dtype=torch.int32, device=device) if n_versions > 1 else None
        if lowram_resid > 0:
            cv = None
            ne = layout.resid_entries(n_kv_heads, batch, cap, lowram_resid)
            pred = torch.zeros(max(1, layout.predictor_elems(rk, batch)), dtype=td, device=device)
            res = torch.zeros((max(1, ne), HEAD_DIM), dtype=td, device=device)
            rsl = torch.full((max(1, ne),), -1, dtype=torch.int32, device=device)
            rno = torch.zeros(max(1, ne), dtype=torch.float32, device=device)
            return cls(dtype, batch, n_q_heads, n_kv_heads, window, cap, rk, rv, bases, ck, cv, ak, av, sk, sv,
                       n_versions, vs, hg, LRKV_VALUES_LOWRAM, lowram_resid, pred, res, rsl, rno)
        return cls(dtype, batch, n_q_heads, n_kv_heads, window, cap, rk, rv, bases, ck, cv, ak, av, sk, sv,
                   n_versions, vs, hg, rope_base=float(rope_base))


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------

def lrkv_compress(layer: Layer, which: int, x, n_tok: int, slot0: int, stream=None):
    """x: device tensor viewed as [batch][n_kv_heads][>= n_tok][128] (any strides,
    last dimension contiguous)."""
    sb, sh, st, si = x.stride()
    assert si == 1
    _check(lib().lrkv_compress(ctypes.byref(layer.struct), which, _ptr(x), sb, sh, st, n_tok, slot0,
                               _stream(stream)), "lrkv_compress")


def lrkv_quantize(layer: Layer, which: int, x, n_tok: int, slot0: int, stream=None):
    """x: float32 device tensor viewed as [batch][n_latent][>= n_tok][>= r]
    (any strides, last dimension contiguous): code rows to quantise into int8
    slots slot0 .. slot0 + n_tok - 1."""
    sb, sh, st, si = x.stride()
    assert si == 1
    _check(lib().lrkv_quantize(ctypes.byref(layer.struct), which, _ptr(x), sb, sh, st, n_tok, slot0,
                               _stream(stream)), "lrkv_quantize")


def lrkv_lowram_workspace_size(layer: Layer) -> int:
    return int(lib().lrkv_lowram_workspace_size(ctypes.byref(layer.struct)))


def lrkv_lowram_fit(layer: Layer, v, n_tok: int, ws=None, stream=None):
    """v: bf16 device tensor viewed as [batch][n_kv_heads][>= n_tok][128], row t the
    value of the token in code slot t (last dimension contiguous).  ``ws``:
    workspace (uint8 device tensor) or None to allocate one."""
    import torch
    sb, sh, st, si = v.stride()
    assert si == 1
    if ws is None:
        ws = torch.empty(max(1, lrkv_lowram_workspace_size(layer)), dtype=torch.uint8, device=v.device)
    _check(lib().lrkv_lowram_fit(ctypes.byref(layer.struct), _ptr(v), sb, sh, st, n_tok, _ptr(ws), ws.numel(),
                                 _stream(stream)), "lrkv_lowram_fit")


def lrkv_oja_workspace_size(layer: Layer) -> int:
    return int(lib().lrkv_oja_workspace_size(ctypes.byref(layer.struct)))


def lrkv_oja_update(layer: Layer, which: int, x, n_tok: int, eta: float, version_in: int, version_out: int,
                    ws=None, stream=None):
    """x: bf16 device tensor viewed as [batch][n_kv_heads][>= n_tok][128] (last
    dimension contiguous).  ``ws``: workspace (uint8 device tensor) or None to
    allocate one."""
    import torch
    sb, sh, st, si = x.stride()
    assert si == 1
    if ws is None:
        ws = torch.empty(max(1, lrkv_oja_workspace_size(layer)), dtype=torch.uint8, device=x.device)
    _check(lib().lrkv_oja_update(ctypes.byref(layer.struct), which, _ptr(x), sb, sh, st, n_tok, eta,
                                 version_in, version_out, _ptr(ws), ws.numel(), _stream(stream)),
           "lrkv_oja_update")


def lrkv_store_anchors(layer: Layer, k, v, pos0: int, n_tok: int, stream=None):
    assert k.stride() == v.stride() and k.stride()[3] == 1
    sb, sh, st, _ = k.stride()
    _check(lib().lrkv_store_anchors(ctypes.byref(layer.struct), _ptr(k), _ptr(v), sb, sh, st, pos0,
                                    n_tok, _stream(stream)), "lrkv_store_anchors")


def lrkv_append(layer: Layer, k_new, v_new, pos: int, stream=None):
    assert k_new.is_contiguous() and v_new.is_contiguous()
    _check(lib().lrkv_append(ctypes.byref(layer.struct), _ptr(k_new), _ptr(v_new), pos,
                             _stream(stream)), "lrkv_append")


def lrkv_decode_workspace_size(layer: Layer, n_splits: int) -> int:
    return int(lib().lrkv_decode_workspace_size(ctypes.byref(layer.struct), n_splits))


def lrkv_decode_auto_splits(layer: Layer, n_ctx: int) -> int:
    return int(lib().lrkv_decode_auto_splits(ctypes.byref(layer.struct), n_ctx))


def workspace(layer: Layer, n_splits: int, device="cuda"):
    """A workspace tensor of the required size (uint8)."""
    import torch
    n = lrkv_decode_workspace_size(layer, n_splits)
    if n == 0:
        raise LrkvError(2, "lrkv_decode_workspace_size")
    return torch.empty(n, dtype=torch.uint8, device=device)


def lrkv_decode_partials(layer: Layer, n_ctx: int, q, sm_scale: float, n_splits: int, ws,
                         ctx_lens=None, stream=None):
    _check(lib().lrkv_decode_partials(ctypes.byref(layer.struct), n_ctx, _ptr(ctx_lens), _ptr(q),
                                      sm_scale, n_splits, _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream)), "lrkv_decode_partials")


def lrkv_decode_combine(layer: Layer, n_ctx: int, n_splits: int, ws, out, ctx_lens=None, stream=None):
    _check(lib().lrkv_decode_combine(ctypes.byref(layer.struct), n_ctx, _ptr(ctx_lens), n_splits,
                                     _ptr(ws), ws.numel() * ws.element_size(), _ptr(out),
                                     _stream(stream)),
           "lrkv_decode_combine")


def lrkv_decode_attn(layer: Layer, n_ctx: int, q, out, sm_scale: float, n_splits: int, ws,
                     ctx_lens=None, stream=None):
    _check(lib().lrkv_decode_attn(ctypes.byref(layer.struct), n_ctx, _ptr(ctx_lens), _ptr(q),
                                  _ptr(out), sm_scale, n_splits, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(stream)),
           "lrkv_decode_attn")


def lrkv_decode_attn_noalloc(layer: Layer, n_ctx: int, q, out, sm_scale: float, n_splits: int, ctx_lens=None,
                             stream=None):
    """lrkv_decode_attn with the split records in the library's per-device array
    (no workspace argument, nothing allocated)."""
    _check(lib().lrkv_decode_attn_noalloc(ctypes.byref(layer.struct), n_ctx, _ptr(ctx_lens), _ptr(q), _ptr(out),
                                          sm_scale, n_splits, _stream(stream)), "lrkv_decode_attn_noalloc")


NOALLOC_CAPACITY = 16 << 20  # bytes of split records lrkv_decode_attn_noalloc holds per device


def lrkv_version() -> int:
    return int(lib().lrkv_version())


def exported_names() -> List[str]:
    return [s[0] for s in SIGNATURES]
