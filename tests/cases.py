"""Shared helpers for the GPU tests: seeded host inputs for one decode step, the
oracle's expected output, and the same inputs laid out on the GPU.

Nothing here feeds a GPU result back into the oracle: codes handed to the GPU
decode come from the oracle's own projection (rounded to storage), and expected
values come only from the oracle.
"""

from __future__ import annotations

import sys
from dataclasses import dataclass
from typing import List, Optional

import numpy as np

import oracle
import synth

D = 128


def to_storage(x, dtype: str) -> np.ndarray:
    """Oracle-side rounding of an exact value to the storage type."""
    if dtype == "bf16":
        return oracle.bf16_round(x)
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def oracle_q8(exact) -> tuple:
    """Int8 codes and scales of exact code rows: the float32 projection, quantised."""
    return oracle.quantize_codes_q8(np.asarray(exact, np.float64).astype(np.float32))


def oracle_q4(exact) -> tuple:
    """4-bit codes and scales of exact code rows: the float32 projection, quantised."""
    return oracle.quantize_codes_q4(np.asarray(exact, np.float64).astype(np.float32))


def oracle_quant(exact, bits: int) -> tuple:
    return oracle_q8(exact) if bits == 8 else oracle_q4(exact)


def code_storage(exact, codes: str) -> np.ndarray:
    """The code values a cache of kind ``codes`` ("f32", "bf16", "q8" or "q4") holds."""
    if codes == "q8":
        return oracle.dequantize_codes_q8(*oracle_q8(exact))
    if codes == "q4":
        return oracle.dequantize_codes_q4(*oracle_q4(exact))
    return to_storage(exact, codes)


@dataclass
class HostCase:
    w: synth.Workload
    n: int                       # context of every row (max when ragged)
    lens: List[int]              # per-row context
    rk: np.ndarray
    rv: np.ndarray
    u_k: list                    # [h] (128, r_k) float64 (exact storage values)
    u_v: list
    k: list                      # [b][h] (n_total, 128) float64 storage values
    v: list
    q: np.ndarray                # (batch, Hq, 128)
    layer: int = 0
    qbits: int = 0               # 8 / 4: quantised codes with per-token scales (bf16 everything else)

    @property
    def codes_kind(self) -> str:
        return f"q{self.qbits}" if self.qbits else self.w.dtype

    @property
    def window(self):
        return self.w.window

    def exact_codes(self, b, h, which, n=None):
        n = self.lens[b] if n is None else n
        pos = oracle.code_positions(n, self.window)
        x = (self.k if which == "k" else self.v)[b][h][pos]
        u = (self.u_k if which == "k" else self.u_v)[h]
        return oracle.oracle_compress(x, u)

    def oracle_codes(self, b, h, which, n=None):
        return code_storage(self.exact_codes(b, h, which, n), self.codes_kind)

    def oracle_anchors(self, b, h, which, n=None):
        n = self.lens[b] if n is None else n
        return (self.k if which == "k" else self.v)[b][h][oracle.anchor_positions(n, self.window)]

    def expected(self, units=None, scale=None) -> np.ndarray:
        """Oracle output (batch, Hq, 128); rows of units not listed stay NaN."""
        w = self.w
        g = w.group
        out = np.full((w.batch, w.n_q_heads, D), np.nan)
        units = units or [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
        for b, h in units:
            rows = slice(h * g, (h + 1) * g)
            out[b, rows] = oracle.oracle_decode_unit(
                self.q[b, rows], self.u_k[h], self.u_v[h],
                self.oracle_codes(b, h, "k"), self.oracle_codes(b, h, "v"),
                self.oracle_anchors(b, h, "k"), self.oracle_anchors(b, h, "v"),
                oracle.default_scale() if scale is None else scale)
        return out


def host_case(w: synth.Workload, n: Optional[int] = None, layer: int = 0, step: int = 0,
              q_scale: float = 1.0, lens: Optional[List[int]] = None, q8: bool = False,
              qbits: int = 0) -> HostCase:
    qbits = 8 if q8 else qbits
    assert not (qbits and w.dtype != "bf16"), "quantised codes come with bf16 bases and anchors"
    n = w.n_ctx if n is None else n
    rk, rv = synth.ranks(w, layer)
    u_k = [synth.basis(w, layer, h, "k", int(rk[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    u_v = [synth.basis(w, layer, h, "v", int(rv[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    k = [[synth.unit_kv(w, layer, h, b, "k").astype(np.float64) for h in range(w.n_kv_heads)]
         for b in range(w.batch)]
    v = [[synth.unit_kv(w, layer, h, b, "v").astype(np.float64) for h in range(w.n_kv_heads)]
         for b in range(w.batch)]
    q = np.stack([synth.queries(w, layer, step, b, q_scale) for b in range(w.batch)]).astype(np.float64)
    lens = [n] * w.batch if lens is None else list(lens)
    return HostCase(w, n, lens, rk, rv, u_k, u_v, k, v, q, layer, qbits)


# ---------------------------------------------------------------------------
# GPU side
# ---------------------------------------------------------------------------

def torch_dtype(dtype: str):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def dev(x, dtype: str):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch_dtype(dtype)).cuda()


def gpu_layer(hc: HostCase, cap: Optional[int] = None, with_codes: bool = True):
    """A Layer whose bases, codes and anchors hold the oracle-made cache of hc."""
    from rank_kv_cache_lrkv_amd import binding as B, layout
    w = hc.w
    W = w.window
    cmax = max(0, hc.n - 1 - W)
    cap = layout.round_cap(cmax) if cap is None else cap
    bases = layout.pack_bases(hc.u_k, hc.u_v)
    dtype = {8: B.LRKV_BF16_Q8, 4: B.LRKV_BF16_Q4}.get(hc.qbits, B.LRKV_F32 if w.dtype == "f32" else B.LRKV_BF16)
    L = B.Layer.allocate(dtype=dtype, batch=w.batch,
                         n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, window=W, cap=cap,
                         rank_k=hc.rk, rank_v=hc.rv, bases=dev(bases, w.dtype))
    if not with_codes:
        return L
    cdt = np.int8 if hc.qbits else np.float32
    ck = np.zeros(max(1, layout.codes_elems(hc.rk, w.batch, cap)), cdt)
    cv = np.zeros(max(1, layout.codes_elems(hc.rv, w.batch, cap)), cdt)
    sk = np.zeros(max(1, layout.scales_elems(w.n_kv_heads, w.batch, cap)), np.float32)
    sv = np.zeros_like(sk)
    ok, ov = layout.code_offsets(hc.rk, w.batch, cap), layout.code_offsets(hc.rv, w.batch, cap)
    ak = np.zeros((w.batch, w.n_kv_heads, 1 + W, D), np.float32)
    av = np.zeros_like(ak)
    for b in range(w.batch):
        nb = hc.lens[b]
        apos = oracle.anchor_positions(nb, W)
        for h in range(w.n_kv_heads):
            for which, flat, off, r, sc in (("k", ck, ok, hc.rk, sk), ("v", cv, ov, hc.rv, sv)):
                base = off[h] + b * cap * int(r[h])
                if hc.qbits:
                    q, s = oracle_quant(hc.exact_codes(b, h, which), hc.qbits)
                    flat[base:base + cap * int(r[h])] = layout.pack_codes(q, cap, which)
                    s0 = layout.scale_offset(h, b, cap, w.batch)
                    sc[s0:s0 + len(s)] = s
                else:
                    codes = hc.oracle_codes(b, h, which)
                    flat[base:base + cap * int(r[h])] = layout.pack_codes(codes.astype(np.float32), cap, which)
            for p in apos:
                s = layout.anchor_slot(int(p), W)
                ak[b, h, s] = hc.k[b][h][p]
                av[b, h, s] = hc.v[b][h][p]
    if hc.qbits:
        import torch
        if hc.qbits == 4:  # element arrays -> bytes, two elements per byte
            ck, cv = layout.pack_nibbles(ck), layout.pack_nibbles(cv)
        L.codes_k.copy_(torch.from_numpy(ck).cuda())
        L.codes_v.copy_(torch.from_numpy(cv).cuda())
        L.scales_k.copy_(torch.from_numpy(sk).cuda())
        L.scales_v.copy_(torch.from_numpy(sv).cuda())
    else:
        L.codes_k.copy_(dev(ck, w.dtype))
        L.codes_v.copy_(dev(cv, w.dtype))
    L.anchor_k.copy_(dev(ak, w.dtype))
    L.anchor_v.copy_(dev(av, w.dtype))
    return L


def gpu_decode(L, hc: HostCase, n_splits: int = 0, scale=None, ragged: bool = False):
    import torch
    from rank_kv_cache_lrkv_amd import binding as B
    S = n_splits or B.lrkv_decode_auto_splits(L, hc.n)
    q = dev(hc.q, hc.w.dtype)
    out = torch.empty((hc.w.batch, hc.w.n_q_heads, D), dtype=torch.float32, device="cuda")
    ws = B.workspace(L, S)
    lens = torch.tensor(hc.lens, dtype=torch.int32, device="cuda") if ragged else None
    B.lrkv_decode_attn(L, hc.n, q, out, oracle.default_scale() if scale is None else scale, S, ws,
                       ctx_lens=lens)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def rel_err(got, want) -> float:
    m = ~np.isnan(want)
    return float(np.max(np.abs(got[m] - want[m])) / np.max(np.abs(want[m])))


def abs_err(got, want) -> float:
    m = ~np.isnan(want)
    return float(np.max(np.abs(got[m] - want[m])))


def check_decode(got, want, dtype: str, label: str):
    """The parity bar: float32 storage max abs error <= 1e-5; bf16 (or int8)
    codes with float32 accumulation max abs error <= 2e-3 of max |out|."""
    assert not np.any(np.isnan(got[~np.isnan(want)])), f"{label}: NaN in GPU output"
    if dtype == "f32":
        e = abs_err(got, want)
        print(f"[parity] {label}: max abs err {e:.3e}", flush=True)
        assert e <= 1e-5, f"{label}: max abs error {e:.3e} > 1e-5"
    else:
        e = rel_err(got, want)
        print(f"[parity] {label}: max err / max|out| {e:.3e}", flush=True)
        assert e <= 2e-3, f"{label}: relative error {e:.3e} > 2e-3"


def announce(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()
