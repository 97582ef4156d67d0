"""Group-head latents on the GPU (Palu abstract: a medium-grained decomposition,
one latent shared by a group of KV heads) against the oracle's group functions.

A layer with head_group = hg keeps one code stream per group of hg consecutive
KV heads, made from their rows joined feature-wise, and every query head reads
its own KV head's slice of the group bases and its own KV head's anchors.

  decode     oracle-made group codes (bf16, int8, 4-bit) so decode is checked
             apart from compress: 2e-3 of max |out|, the bar of bf16 codes
  compress   lrkv_compress from bf16 rows: every code within the float32
             accumulation bound over hg * 128 features (quantised: within one
             step, >= 99.9% identical), as for single heads
  append     prefill compression, anchors, appends and decode steps against the
             oracle's own cache
  full size  the 32K Llama-3.1-8B-shaped layer, sampled units
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import D, announce, check_decode, code_storage, dev, oracle_quant
from rank_kv_cache_lrkv_amd import binding as B, layout

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
DTYPE = {0: B.LRKV_BF16, 8: B.LRKV_BF16_Q8, 4: B.LRKV_BF16_Q4}
QMAX = {8: 127, 4: 7}


@dataclass
class GroupCase:
    w: synth.Workload
    hg: int
    n: int
    lens: List[int]
    rk: np.ndarray               # per latent group
    rv: np.ndarray
    u_k: list                    # [g] (hg * 128, r_k) float64 storage values
    u_v: list
    k: list                      # [b][h] (n_total, 128) float64 storage values, per KV head
    v: list
    q: np.ndarray                # (batch, Hq, 128)
    qbits: int = 0

    @property
    def n_lat(self) -> int:
        return self.w.n_kv_heads // self.hg

    @property
    def kind(self) -> str:
        return f"q{self.qbits}" if self.qbits else "bf16"

    def joined(self, b, g, which, pos):
        """(hg, len(pos), 128) rows of the group's KV heads at positions pos."""
        src = self.k if which == "k" else self.v
        return np.stack([src[b][g * self.hg + j][pos] for j in range(self.hg)])

    def exact_codes(self, b, g, which, n=None):
        n = self.lens[b] if n is None else n
        u = (self.u_k if which == "k" else self.u_v)[g]
        return oracle.oracle_compress_group(self.joined(b, g, which, oracle.code_positions(n, self.w.window)), u)

    def expected(self, units=None, n=None, q=None) -> np.ndarray:
        w, hg = self.w, self.hg
        gk = w.group
        G = gk * hg
        q = self.q if q is None else q
        out = np.full((w.batch, w.n_q_heads, D), np.nan)
        units = units or [(b, g) for b in range(w.batch) for g in range(self.n_lat)]
        for b, g in units:
            nb = self.lens[b] if n is None else n
            apos = oracle.anchor_positions(nb, w.window)
            ck = code_storage(self.exact_codes(b, g, "k", nb), self.kind)
            cv = code_storage(self.exact_codes(b, g, "v", nb), self.kind)
            rows = slice(g * G, (g + 1) * G)
            out[b, rows] = oracle.oracle_decode_group(
                q[b, rows], [i // gk for i in range(G)], self.u_k[g], self.u_v[g], ck, cv,
                list(self.joined(b, g, "k", apos)), list(self.joined(b, g, "v", apos)), oracle.default_scale())
        return out


def group_case(w, hg, layer=0, step=0, lens=None, qbits=0, q_scale=1.0) -> GroupCase:
    n_lat = w.n_kv_heads // hg
    rk = np.full(n_lat, w.rank_k, np.int32)
    rv = np.full(n_lat, w.rank_v, np.int32)
    u_k = [synth.group_basis(w, layer, g, hg, "k", w.rank_k).astype(np.float64) for g in range(n_lat)]
    u_v = [synth.group_basis(w, layer, g, hg, "v", w.rank_v).astype(np.float64) for g in range(n_lat)]
    k = [[synth.unit_kv(w, layer, h, b, "k").astype(np.float64) for h in range(w.n_kv_heads)]
         for b in range(w.batch)]
    v = [[synth.unit_kv(w, layer, h, b, "v").astype(np.float64) for h in range(w.n_kv_heads)]
         for b in range(w.batch)]
    q = np.stack([synth.queries(w, layer, step, b, q_scale) for b in range(w.batch)]).astype(np.float64)
    lens = [w.n_ctx] * w.batch if lens is None else list(lens)
    return GroupCase(w, hg, w.n_ctx, lens, rk, rv, u_k, u_v, k, v, q, qbits)


def allocate(gc: GroupCase, cap: int):
    w = gc.w
    return B.Layer.allocate(dtype=DTYPE[gc.qbits], batch=w.batch, n_q_heads=w.n_q_heads,
                            n_kv_heads=w.n_kv_heads, window=w.window, cap=cap, rank_k=gc.rk, rank_v=gc.rv,
                            bases=dev(layout.pack_bases(gc.u_k, gc.u_v), "bf16"), head_group=gc.hg)


def gpu_group_layer(gc: GroupCase):
    """A layer holding the oracle-made group cache of gc."""
    w, Wn = gc.w, gc.w.window
    cap = layout.round_cap(max(0, gc.n - 1 - Wn))
    L = allocate(gc, cap)
    cdt = np.int8 if gc.qbits else np.float32
    ck = np.zeros(max(1, layout.codes_elems(gc.rk, w.batch, cap)), cdt)
    cv = np.zeros(max(1, layout.codes_elems(gc.rv, w.batch, cap)), cdt)
    sk = np.zeros(max(1, layout.scales_elems(gc.n_lat, w.batch, cap)), np.float32)
    sv = np.zeros_like(sk)
    ok, ov = layout.code_offsets(gc.rk, w.batch, cap), layout.code_offsets(gc.rv, w.batch, cap)
    ak = np.zeros((w.batch, w.n_kv_heads, 1 + Wn, D), np.float32)
    av = np.zeros_like(ak)
    for b in range(w.batch):
        for g in range(gc.n_lat):
            for which, flat, off, r, sc in (("k", ck, ok, gc.rk, sk), ("v", cv, ov, gc.rv, sv)):
                base = off[g] + b * cap * int(r[g])
                exact = gc.exact_codes(b, g, which)
                if gc.qbits:
                    qv, s = oracle_quant(exact, gc.qbits)
                    flat[base:base + cap * int(r[g])] = layout.pack_codes(qv, cap, which)
                    s0 = layout.scale_offset(g, b, cap, w.batch)
                    sc[s0:s0 + len(s)] = s
                else:
                    codes = code_storage(exact, "bf16").astype(np.float32)
                    flat[base:base + cap * int(r[g])] = layout.pack_codes(codes, cap, which)
        for p in oracle.anchor_positions(gc.lens[b], Wn):
            s = layout.anchor_slot(int(p), Wn)
            for h in range(w.n_kv_heads):
                ak[b, h, s] = gc.k[b][h][p]
                av[b, h, s] = gc.v[b][h][p]
    if gc.qbits:
        if gc.qbits == 4:
            ck, cv = layout.pack_nibbles(ck), layout.pack_nibbles(cv)
        L.codes_k.copy_(torch.from_numpy(ck).cuda())
        L.codes_v.copy_(torch.from_numpy(cv).cuda())
        L.scales_k.copy_(torch.from_numpy(sk).cuda())
        L.scales_v.copy_(torch.from_numpy(sv).cuda())
    else:
        L.codes_k.copy_(dev(ck, "bf16"))
        L.codes_v.copy_(dev(cv, "bf16"))
    L.anchor_k.copy_(dev(ak, "bf16"))
    L.anchor_v.copy_(dev(av, "bf16"))
    return L


def run_decode(L, w, n, q_np, S=0, lens=None):
    S = S or B.lrkv_decode_auto_splits(L, n)
    q = dev(q_np, "bf16")
    out = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device="cuda")
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda") if lens is not None else None
    B.lrkv_decode_attn(L, n, q, out, oracle.default_scale(), S, B.workspace(L, S), ctx_lens=cl)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


# ---------------------------------------------------------------------------
# decode on oracle-made group codes
# ---------------------------------------------------------------------------

LLAMA = W["llama31_8b_32k"]
QWEN = W["qwen3_1p7b_4k"]
BASE = QWEN.scaled(batch=2, n_q_heads=8, n_kv_heads=4, window=16)

DECODE = [
    # label, workload, head_group, n_splits, ragged lengths
    ("llama_hg2_n3000_s32", LLAMA.scaled(batch=1, n_ctx=3000), 2, 32, None),
    ("llama_hg4_n1000", LLAMA.scaled(batch=2, n_ctx=1000), 4, 0, None),
    ("qwen_hg8_n700", QWEN.scaled(batch=2, n_ctx=700), 8, 0, None),
    ("hg2_ranks_128", BASE.scaled(n_ctx=500, rank_k=128, rank_v=128), 2, 0, None),
    ("hg2_ranks_16", BASE.scaled(n_ctx=500, rank_k=16, rank_v=16), 2, 0, None),
    ("hg4_g1", BASE.scaled(n_q_heads=4, n_ctx=400), 4, 0, None),
    ("hg2_n1", BASE.scaled(n_ctx=1), 2, 0, None),
    ("hg2_n_window_plus_2", BASE.scaled(n_ctx=18), 2, 0, None),
    ("hg2_window0", BASE.scaled(window=0, n_ctx=300), 2, 0, None),
    ("hg4_wide_window_s8", BASE.scaled(window=64, n_ctx=200), 4, 8, None),   # 4 x 65 anchor rows over 8 splits
    ("hg2_one_split", BASE.scaled(n_ctx=900), 2, 1, None),
    ("hg2_empty_splits", BASE.scaled(n_ctx=17 + 40), 2, 16, None),
    ("hg2_many_splits", BASE.scaled(n_ctx=700), 2, 300, None),
    ("hg2_ragged", BASE.scaled(batch=5, n_ctx=800), 2, 0, [800, 1, 17, 18, 433]),
]


@pytest.mark.parametrize("label,w,hg,S,lens", DECODE, ids=[d[0] for d in DECODE])
def test_group_decode(label, w, hg, S, lens):
    announce(f"group decode {label}: hg {hg} batch {w.batch} n {w.n_ctx} S {S}")
    gc = group_case(w, hg, lens=lens)
    got = run_decode(gpu_group_layer(gc), w, gc.n, gc.q, S, lens)
    check_decode(got, gc.expected(), "bf16", f"group_{label}")


Q_DECODE = [d for d in DECODE if d[0] in ("llama_hg2_n3000_s32", "qwen_hg8_n700", "hg2_ranks_128",
                                           "hg4_wide_window_s8", "hg2_ragged")]


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("label,w,hg,S,lens", Q_DECODE, ids=[d[0] for d in Q_DECODE])
def test_group_decode_q(label, w, hg, S, lens, bits):
    announce(f"group decode {bits}-bit {label}: hg {hg} batch {w.batch} n {w.n_ctx} S {S}")
    gc = group_case(w, hg, lens=lens, qbits=bits)
    got = run_decode(gpu_group_layer(gc), w, gc.n, gc.q, S, lens)
    check_decode(got, gc.expected(), "bf16", f"group_q{bits}_{label}")


def test_group_decode_peaky():
    w = BASE.scaled(n_ctx=900)
    gc = group_case(w, 2, q_scale=8.0)
    announce("group decode peaky q x8")
    check_decode(run_decode(gpu_group_layer(gc), w, gc.n, gc.q), gc.expected(), "bf16", "group_peaky")


# ---------------------------------------------------------------------------
# compress from bf16 rows
# ---------------------------------------------------------------------------

def bf16_ulp(x):
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def read_group_codes(L, which, b, g, n, slot0=0):
    """(codes (n, r) float64 or int, scales (n,) or None) of slots slot0 ..."""
    ranks = L.rank_k if which == "k" else L.rank_v
    r = int(ranks[g])
    off = int(layout.code_offsets(ranks, L.batch, L.cap)[g]) + b * L.cap * r
    buf = L.codes_k if which == "k" else L.codes_v
    if L.dtype == B.LRKV_BF16_Q4:
        flat = layout.unpack_nibbles(buf[off // 2:(off + L.cap * r) // 2].cpu().numpy())
    elif L.dtype == B.LRKV_BF16_Q8:
        flat = buf[off:off + L.cap * r].cpu().numpy()
    else:
        flat = buf[off:off + L.cap * r].float().cpu().numpy().astype(np.float64)
    codes = layout.unpack_codes(flat, slot0 + n, r, which)[slot0:]
    if L.dtype == B.LRKV_BF16:
        return codes, None
    s0 = layout.scale_offset(g, b, L.cap, L.batch)
    return codes, (L.scales_k if which == "k" else L.scales_v)[s0 + slot0:s0 + slot0 + n].cpu().numpy()


def check_group_codes(got, sc, x, u, bits, label):
    """x (t, hg * 128) joined rows, u (hg * 128, r).  The float32 accumulation
    bound is gamma_m sum |x_i u_i| with m = hg * 128 terms."""
    exact = x @ u
    if not got.size:
        return
    m = x.shape[1]
    uu = 2.0 ** -24
    acc = (m * uu / (1 - m * uu)) * (np.abs(x) @ np.abs(u))
    if bits == 0:
        bound = acc + 0.5 * bf16_ulp(np.abs(exact) + acc)
        worst = float(np.max(np.abs(got - exact) / bound))
        equal = float(np.mean(got == oracle.bf16_round(exact)))
        print(f"[parity] {label}: compress worst {worst:.3f} of bound, bit-equal {equal:.5f}", flush=True)
        assert worst <= 1.0, (label, worst)
        assert equal >= 0.99, (label, equal)
        return
    q_want, s_want = oracle_quant(exact, bits)
    s_tol = np.max(acc, axis=1) / QMAX[bits] + 2 * np.spacing(s_want.astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(sc.astype(np.float64) - s_want) <= s_tol), label
    dq = np.abs(got.astype(np.int32) - q_want.astype(np.int32))
    equal = float(np.mean(dq == 0))
    print(f"[parity] {label}: {bits}-bit codes equal {equal:.5f}, max |dq| {int(dq.max())}", flush=True)
    assert dq.max() <= 1, label
    assert equal >= 0.999, (label, equal)


def rows_tensor(gc, which, n):
    src = gc.k if which == "k" else gc.v
    a = np.stack([np.stack([src[b][h][:n] for h in range(gc.w.n_kv_heads)]) for b in range(gc.w.batch)])
    return dev(a, "bf16")


COMPRESS = [
    ("llama_hg2_n1000", LLAMA.scaled(batch=2, n_ctx=1000), 2),
    ("qwen_hg8_n333", QWEN.scaled(batch=1, n_ctx=333), 8),
    ("hg4_ranks_128_16", BASE.scaled(n_ctx=290, rank_k=128, rank_v=16), 4),
]


@pytest.mark.parametrize("bits", [0, 8, 4])
@pytest.mark.parametrize("label,w,hg", COMPRESS, ids=[c[0] for c in COMPRESS])
@pytest.mark.parametrize("slot0", [0, 3])
def test_group_compress(label, w, hg, slot0, bits):
    announce(f"group compress {label} bits {bits} slot0 {slot0}")
    gc = group_case(w, hg, qbits=bits)
    c = max(0, gc.n - 1 - w.window)
    L = allocate(gc, layout.round_cap(c + slot0))
    for which in "kv":
        B.lrkv_compress(L, 0 if which == "k" else 1, rows_tensor(gc, which, gc.n)[:, :, 1:1 + c], c, slot0)
    torch.cuda.synchronize()
    for which in "kv":
        for b in range(w.batch):
            for g in range(gc.n_lat):
                got, sc = read_group_codes(L, which, b, g, c, slot0)
                x = np.concatenate(list(gc.joined(b, g, which, np.arange(1, 1 + c))), axis=1)
                u = (gc.u_k if which == "k" else gc.u_v)[g]
                check_group_codes(got, sc, x, u, bits, f"{label}/{which}/b{b}g{g}/s{slot0}")


# ---------------------------------------------------------------------------
# end to end: prefill compression, anchors and appends
# ---------------------------------------------------------------------------

def prefill(gc, n, extra=0):
    w = gc.w
    c = max(0, n - 1 - w.window)
    L = allocate(gc, layout.round_cap(c + extra))
    K, V = rows_tensor(gc, "k", w.n_total), rows_tensor(gc, "v", w.n_total)
    B.lrkv_compress(L, 0, K[:, :, 1:], c, 0)
    B.lrkv_compress(L, 1, V[:, :, 1:], c, 0)
    B.lrkv_store_anchors(L, K[:, :, 0:1], V[:, :, 0:1], 0, 1)
    lo = max(1, n - w.window)
    B.lrkv_store_anchors(L, K[:, :, lo:n], V[:, :, lo:n], lo, n - lo)
    return L, K, V


@pytest.mark.parametrize("bits", [0, 8, 4])
@pytest.mark.parametrize("window", [0, 1, 16])
def test_group_decode_steps_with_append(window, bits):
    w = LLAMA.scaled(batch=2, n_ctx=60, n_steps=40, window=window)
    announce(f"group e2e append steps W={window} bits {bits}")
    gc = group_case(w, 2, layer=3, qbits=bits)
    L, K, V = prefill(gc, w.n_ctx, extra=w.n_steps)
    for t in range(1, w.n_steps + 1):
        pos = w.n_ctx + t - 1
        B.lrkv_append(L, K[:, :, pos].contiguous(), V[:, :, pos].contiguous(), pos)
        n = pos + 1
        q = np.stack([synth.queries(w, 3, t, b) for b in range(w.batch)]).astype(np.float64)
        got = run_decode(L, w, n, q)
        if t in (1, 2, w.window + 1, w.window + 2, w.n_steps) or t % 9 == 0:
            check_decode(got, gc.expected(n=n, q=q), "bf16", f"group_q{bits}_append_W{window}_t{t}")


def test_group_full_size_llama_32k_sampled():
    """The 32K Llama-3.1-8B-shaped layer with pairs of KV heads sharing codes
    (32 splits): GPU prefill compression, then one decode, sampled units."""
    w = LLAMA
    gc = group_case(w, 2)
    announce(f"group full size llama31_8b_32k: hg 2 batch {w.batch} n {w.n_ctx}")
    L, _, _ = prefill(gc, w.n_ctx)
    got = run_decode(L, w, w.n_ctx, gc.q, 32)
    assert np.all(np.isfinite(got))
    units = [(0, 0), (w.batch // 2, 1), (w.batch - 1, gc.n_lat - 1)]
    check_decode(got, gc.expected(units), "bf16", "group_full_llama31_8b_32k")
