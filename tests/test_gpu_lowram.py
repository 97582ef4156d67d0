"""LowRAM value amortisation on the GPU (LowRAM abstract: values predicted from
the keys by a per-head predictor fitted at test time, residuals kept for the
worst-predicted tokens) against the oracle (oracle.lowram_* and
oracle_decode_lowram).

  fit      lrkv_lowram_fit on oracle-made key codes and bf16 values: predictions
           C M within 2e-3 of the oracle's (relative Frobenius; M itself is as
           ill-conditioned as C^T C, the predictions are not), the kept slots a
           top-R of every block under the oracle's norms up to the float32 error,
           kept residual rows within the same bound
  decode   an oracle-made LowRAM cache (codes, predictor, kept residual rows):
           2e-3 of max |out|, the bar of bf16 codes
  e2e      GPU prefill compression, anchors, fit, appends and decode steps
           against the oracle's own chain from the same rows: the device's choice
           of kept slots checked to be a valid top R, then the oracle decodes with
           exactly those slots, at 2e-3 of max |out|
  full     the 32K Llama-3.1-8B-shaped layer, sampled units
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import D, announce, check_decode, dev
from rank_kv_cache_lrkv_amd import binding as B, layout

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
LLAMA = W["llama31_8b_32k"].scaled(v_from_k=0.8)
QWEN = W["qwen3_1p7b_4k"].scaled(v_from_k=0.8)
BASE = QWEN.scaled(batch=2, n_q_heads=8, n_kv_heads=2, window=16)
RV_DUMMY = 16  # rank_v only lays out the bases here (no value codes)


@dataclass
class LRCase:
    w: synth.Workload
    R: int
    n: int
    lens: List[int]
    rk: np.ndarray
    u_k: list              # [h] (128, r_k) float64 storage values
    k: list                # [b][h] (n_total, 128)
    v: list
    q: np.ndarray          # (batch, Hq, 128)

    def codes(self, b, h, n=None):
        n = self.lens[b] if n is None else n
        pos = oracle.code_positions(n, self.w.window)
        return oracle.bf16_round(oracle.oracle_compress(self.k[b][h][pos], self.u_k[h]))

    def values(self, b, h, n=None):
        n = self.lens[b] if n is None else n
        return self.v[b][h][oracle.code_positions(n, self.w.window)]

    def cache(self, b, h, n_fit=None, n=None):
        """The oracle's cache of (b, h): codes, M fitted on the first n_fit code
        slots, kept slots (the prefill choice, then the blockwise rule over every
        slot up to n: the same set), residual rows of every slot."""
        ck, vv = self.codes(b, h, n), self.values(b, h, n)
        nf = len(ck) if n_fit is None else n_fit
        m, _, _ = oracle.lowram_prefill(ck[:nf], vv[:nf], self.R)
        e = oracle.lowram_residuals(ck, vv, m)
        kept = oracle.lowram_select(np.sum(e * e, axis=1), self.R)
        return ck, m, kept, oracle.bf16_round(e), np.sum(e * e, axis=1)

    def expected(self, units=None, n=None, q=None, n_fit=None) -> np.ndarray:
        w = self.w
        g = w.group
        q = self.q if q is None else q
        out = np.full((w.batch, w.n_q_heads, D), np.nan)
        units = units or [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
        for b, h in units:
            nb = self.lens[b] if n is None else n
            apos = oracle.anchor_positions(nb, w.window)
            ck, m, kept, e, _ = self.cache(b, h, n_fit, nb)
            rows = slice(h * g, (h + 1) * g)
            out[b, rows] = oracle.oracle_decode_lowram(q[b, rows], self.u_k[h], m, ck, kept, e,
                                                       self.k[b][h][apos], self.v[b][h][apos],
                                                       oracle.default_scale())
        return out


def lr_case(w, R, layer=0, step=0, lens=None, q_scale=1.0) -> LRCase:
    rk, _ = synth.ranks(w, layer)
    u_k = [synth.basis(w, layer, h, "k", int(rk[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    k = [[synth.unit_kv(w, layer, h, b, "k").astype(np.float64) for h in range(w.n_kv_heads)]
         for b in range(w.batch)]
    v = [[synth.unit_kv(w, layer, h, b, "v").astype(np.float64) for h in range(w.n_kv_heads)]
         for b in range(w.batch)]
    q = np.stack([synth.queries(w, layer, step, b, q_scale) for b in range(w.batch)]).astype(np.float64)
    lens = [w.n_ctx] * w.batch if lens is None else list(lens)
    return LRCase(w, R, w.n_ctx, lens, rk, u_k, k, v, q)


def allocate(c: LRCase, cap: int):
    w = c.w
    rv = np.full(w.n_kv_heads, RV_DUMMY, np.int32)
    bases = layout.pack_bases(c.u_k, [np.zeros((D, RV_DUMMY))] * w.n_kv_heads)
    return B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                            window=w.window, cap=cap, rank_k=c.rk, rank_v=rv, bases=dev(bases, "bf16"),
                            lowram_resid=c.R)


def gpu_lr_layer(c: LRCase):
    """A layer holding the oracle-made LowRAM cache of c."""
    w, Wn = c.w, c.w.window
    cap = layout.round_cap(max(0, c.n - 1 - Wn))
    L = allocate(c, cap)
    ck = np.zeros(max(1, layout.codes_elems(c.rk, w.batch, cap)), np.float32)
    pred = np.zeros(max(1, layout.predictor_elems(c.rk, w.batch)), np.float32)
    ne = layout.resid_entries(w.n_kv_heads, w.batch, cap, c.R)
    rows = np.zeros((max(1, ne), D), np.float32)
    slots = np.full(max(1, ne), -1, np.int32)
    norms = np.zeros(max(1, ne), np.float32)
    ak = np.zeros((w.batch, w.n_kv_heads, 1 + Wn, D), np.float32)
    av = np.zeros_like(ak)
    off = layout.code_offsets(c.rk, w.batch, cap)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            r = int(c.rk[h])
            codes, m, kept, e, sq = c.cache(b, h)
            base = off[h] + b * cap * r
            ck[base:base + cap * r] = layout.pack_codes(codes.astype(np.float32), cap, "k")
            p0 = layout.predictor_offset(c.rk, w.batch, h, b)
            pred[p0:p0 + r * D] = m.ravel()
            count = {}
            for t in kept:
                blk = int(t) // 32
                i = count.get(blk, 0)
                count[blk] = i + 1
                ei = layout.resid_entry(h, b, blk, i, w.batch, cap, c.R)
                rows[ei], slots[ei], norms[ei] = e[t], int(t) % 32, sq[t]
        for p in oracle.anchor_positions(c.lens[b], Wn):
            s = layout.anchor_slot(int(p), Wn)
            for h in range(w.n_kv_heads):
                ak[b, h, s] = c.k[b][h][p]
                av[b, h, s] = c.v[b][h][p]
    L.codes_k.copy_(dev(ck, "bf16"))
    L.predictor.copy_(dev(pred, "bf16"))
    L.resid.copy_(dev(rows, "bf16"))
    L.resid_slot.copy_(torch.from_numpy(slots).cuda())
    L.resid_norm.copy_(torch.from_numpy(norms).cuda())
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
# decode on oracle-made LowRAM caches
# ---------------------------------------------------------------------------

DECODE = [
    # label, workload, R, n_splits, ragged lengths
    ("llama_n3000_s32_r4", LLAMA.scaled(batch=1, n_ctx=3000), 4, 32, None),
    ("qwen_n1000_r8", QWEN.scaled(batch=2, n_ctx=1000), 8, 0, None),
    ("hc_n777_r1", W["llama31_8b_hc_8k"].scaled(batch=3, n_ctx=777, v_from_k=0.5), 1, 0, None),
    ("mixed_ranks_n2000_r4", W["llama31_8b_32layer"].scaled(batch=2, n_ctx=2000, n_steps=0, v_from_k=0.8),
     4, 0, None),
    ("ranks_16_48_96_128_r3", BASE.scaled(n_kv_heads=4, n_q_heads=8, n_ctx=500, mixed_ranks=True,
                                          rank_k_choices=(16, 48, 96, 128)), 3, 0, None),
    ("independent_values_r8", BASE.scaled(n_ctx=700, v_from_k=0.0), 8, 0, None),
    ("n1", BASE.scaled(n_ctx=1), 4, 0, None),
    ("n_window_plus_2", BASE.scaled(n_ctx=18), 4, 0, None),
    ("window0", BASE.scaled(window=0, n_ctx=300), 4, 0, None),
    ("empty_splits", BASE.scaled(n_ctx=17 + 40), 4, 16, None),
    ("many_splits", BASE.scaled(n_ctx=700), 4, 300, None),
    ("one_split", BASE.scaled(n_ctx=900), 4, 1, None),
    ("gqa_g16", BASE.scaled(n_q_heads=32, n_ctx=400), 4, 0, None),
    ("ragged", BASE.scaled(batch=5, n_ctx=800), 4, 0, [800, 1, 17, 18, 433]),
]


@pytest.mark.parametrize("label,w,R,S,lens", DECODE, ids=[d[0] for d in DECODE])
def test_lowram_decode(label, w, R, S, lens):
    announce(f"lowram decode {label}: R {R} batch {w.batch} n {w.n_ctx} S {S}")
    c = lr_case(w, R, lens=lens)
    got = run_decode(gpu_lr_layer(c), w, c.n, c.q, S, lens)
    check_decode(got, c.expected(), "bf16", f"lowram_{label}")


def test_lowram_decode_peaky():
    w = BASE.scaled(n_ctx=900)
    c = lr_case(w, 4, q_scale=8.0)
    announce("lowram decode peaky q x8")
    check_decode(run_decode(gpu_lr_layer(c), w, c.n, c.q), c.expected(), "bf16", "lowram_peaky")


# ---------------------------------------------------------------------------
# the fit
# ---------------------------------------------------------------------------

def read_lr(L, c, b, h, n_tok):
    """(M (r, 128), kept slots, residual rows by slot, norms by slot) from the device."""
    w = c.w
    r = int(c.rk[h])
    p0 = layout.predictor_offset(c.rk, w.batch, h, b)
    m = L.predictor[p0:p0 + r * D].float().cpu().numpy().astype(np.float64).reshape(r, D)
    slots = L.resid_slot.cpu().numpy()
    rows = L.resid.float().cpu().numpy().astype(np.float64)
    norms = L.resid_norm.cpu().numpy()
    kept, e, sq = [], {}, {}
    for blk in range((n_tok + 31) // 32):
        for i in range(c.R):
            ei = layout.resid_entry(h, b, blk, i, w.batch, L.cap, c.R)
            if slots[ei] >= 0:
                t = blk * 32 + int(slots[ei])
                kept.append(t)
                e[t], sq[t] = rows[ei], float(norms[ei])
    return m, np.array(sorted(kept)), e, sq


FIT = [
    ("qwen_n1000_r4", QWEN.scaled(batch=2, n_ctx=1000), 4),
    ("llama_n2000_r8", LLAMA.scaled(batch=1, n_ctx=2000), 8),
    ("ranks_16_48_96_128_r2", BASE.scaled(n_kv_heads=4, n_q_heads=8, n_ctx=333, mixed_ranks=True,
                                          rank_k_choices=(16, 48, 96, 128)), 2),
    ("independent_values_r1", BASE.scaled(n_ctx=500, v_from_k=0.0), 1),
]


@pytest.mark.parametrize("label,w,R", FIT, ids=[f[0] for f in FIT])
def test_lowram_fit(label, w, R):
    announce(f"lowram fit {label}: R {R}")
    c = lr_case(w, R)
    nc = max(0, c.n - 1 - w.window)
    L = allocate(c, layout.round_cap(nc))
    ck = np.zeros(max(1, layout.codes_elems(c.rk, w.batch, L.cap)), np.float32)
    off = layout.code_offsets(c.rk, w.batch, L.cap)
    vv = np.zeros((w.batch, w.n_kv_heads, nc, D), np.float32)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            r = int(c.rk[h])
            ck[off[h] + b * L.cap * r:off[h] + (b + 1) * L.cap * r] = \
                layout.pack_codes(c.codes(b, h).astype(np.float32), L.cap, "k")
            vv[b, h] = c.values(b, h)
    L.codes_k.copy_(dev(ck, "bf16"))
    B.lrkv_lowram_fit(L, dev(vv, "bf16"), nc)
    torch.cuda.synchronize()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            codes, m_or, _, _, sq_or = c.cache(b, h)
            m, kept, e, sq = read_lr(L, c, b, h, nc)
            vals = c.values(b, h)
            scale = np.linalg.norm(vals)
            pred_err = np.linalg.norm(codes @ (m - m_or)) / scale
            equal = float(np.mean(m == m_or))
            print(f"[parity] {label}/b{b}h{h}: predictions {pred_err:.2e} of |V|, M bit-equal {equal:.3f}",
                  flush=True)
            assert pred_err <= 2e-3, (label, b, h, pred_err)
            # every block keeps min(R, its slots) slots, a top R under the oracle's
            # norms up to the norm change the predictor's rounding can cause
            e_or = oracle.lowram_residuals(codes, vals, m_or)
            tol = 2 * np.sqrt(sq_or) * np.linalg.norm(codes @ (m - m_or), axis=1) + 1e-6 * sq_or.max()
            ks = set(kept.tolist())
            for b0 in range(0, nc, 32):
                blk = list(range(b0, min(b0 + 32, nc)))
                k_in = [t for t in blk if t in ks]
                assert len(k_in) == min(R, len(blk)), (label, b, h, b0)
                drop = [t for t in blk if t not in ks]
                if k_in and drop:
                    worst_kept = min(sq_or[t] + tol[t] for t in k_in)
                    best_dropped = max(sq_or[t] - tol[t] for t in drop)
                    assert worst_kept >= best_dropped, (label, b, h, b0)
            for t in kept:
                d = np.linalg.norm(e[t] - e_or[t])
                bound = np.linalg.norm(codes[t] @ (m - m_or)) + 2 ** -8 * np.abs(e_or[t]).max() * np.sqrt(D) \
                    + 1e-5 * np.linalg.norm(vals[t])
                assert d <= bound, (label, b, h, int(t), d, bound)
                assert abs(sq[t] - np.sum(e_or[t] ** 2)) <= tol[t] + 1e-3 * sq_or[t], (label, b, h, int(t))


# ---------------------------------------------------------------------------
# end to end: compress, anchors, fit, appends, decode
#
# The kept slots are a choice by norm, taken in float32 on the device from its
# own predictor: where norms near a block's cut lie within the float32 error of
# each other, either choice is valid.  So each device choice is first checked to
# be a top R of every block under the oracle's norms within MARGIN; then the
# oracle decodes with exactly the slots the device kept (its own predictor and
# residual rows) and the output must match within the plain decode bar.
# ---------------------------------------------------------------------------

MARGIN = 2e-3  # of the block's largest squared norm


def device_kept(slots, c, L, b, h, n_slots):
    """The code slots the device keeps residual rows for in (b, h)."""
    kept = []
    for blk in range((n_slots + 31) // 32):
        for i in range(c.R):
            s_ = int(slots[layout.resid_entry(h, b, blk, i, c.w.batch, L.cap, c.R)])
            if s_ >= 0:
                kept.append(blk * 32 + s_)
    return np.array(sorted(kept), dtype=np.int64)


def check_device_choice(L, c, units, n_fit, n):
    slots = L.resid_slot.cpu().numpy()
    for b, h in units:
        ck, _, _, _, sq = c.cache(b, h, n_fit, n)
        ns = len(ck)
        kept = set(device_kept(slots, c, L, b, h, ns).tolist())
        for blk in range((ns + 31) // 32):
            slots_blk = list(range(blk * 32, min(blk * 32 + 32, ns)))
            got = {t for t in kept if blk * 32 <= t < blk * 32 + 32}
            assert got <= set(slots_blk) and len(got) == min(c.R, len(slots_blk)), (b, h, blk, sorted(got))
            drop = [t for t in slots_blk if t not in got]
            if got and drop:
                top = max(sq[t] for t in slots_blk)
                assert min(sq[t] for t in got) >= max(sq[t] for t in drop) - MARGIN * top, (b, h, blk)
    return slots


def compare_on_device_choice(got, c, units, n, q, n_fit, L, label):
    """The device's kept slots must be a valid top R (within MARGIN); the oracle
    then decodes with those slots and the output must be within 2e-3 of max |out|."""
    w = c.w
    g = w.group
    slots = check_device_choice(L, c, units, n_fit, n)
    want = np.full((w.batch, w.n_q_heads, D), np.nan)
    apos = oracle.anchor_positions(n, w.window)
    n_diff = 0
    for b, h in units:
        ck, m, kept_or, e, _ = c.cache(b, h, n_fit, n)
        kept = device_kept(slots, c, L, b, h, len(ck))
        n_diff += len(set(kept.tolist()) ^ set(np.asarray(kept_or).tolist())) // 2
        rows = slice(h * g, (h + 1) * g)
        want[b, rows] = oracle.oracle_decode_lowram(q[b, rows], c.u_k[h], m, ck, kept, e, c.k[b][h][apos],
                                                    c.v[b][h][apos], oracle.default_scale())
    print(f"[parity] {label}: {n_diff} kept slots differ from the oracle's own choice", flush=True)
    check_decode(got, want, "bf16", label)


def rows_tensor(c, which, n):
    src = c.k if which == "k" else c.v
    a = np.stack([np.stack([src[b][h][:n] for h in range(c.w.n_kv_heads)]) for b in range(c.w.batch)])
    return dev(a, "bf16")


def prefill(c, n, extra=0):
    w = c.w
    nc = max(0, n - 1 - w.window)
    L = allocate(c, layout.round_cap(nc + extra))
    K, V = rows_tensor(c, "k", w.n_total), rows_tensor(c, "v", w.n_total)
    B.lrkv_compress(L, 0, K[:, :, 1:], nc, 0)
    if nc > 0:
        B.lrkv_lowram_fit(L, V[:, :, 1:], nc)
    B.lrkv_store_anchors(L, K[:, :, 0:1], V[:, :, 0:1], 0, 1)
    lo = max(1, n - w.window)
    B.lrkv_store_anchors(L, K[:, :, lo:n], V[:, :, lo:n], lo, n - lo)
    return L, K, V, nc


@pytest.mark.parametrize("R", [1, 4])
@pytest.mark.parametrize("window", [0, 1, 16])
def test_lowram_decode_steps_with_append(window, R):
    # a prompt of several times rank_k tokens: the least-squares fit is well posed
    # (with fewer code rows than rank_k the predictor is fixed only by the tiny
    # ridge, and float32 and float64 solves part ways)
    w = LLAMA.scaled(batch=2, n_ctx=400, n_steps=48, window=window)
    announce(f"lowram e2e append steps W={window} R={R}")
    c = lr_case(w, R, layer=3)
    L, K, V, nfit = prefill(c, w.n_ctx, extra=w.n_steps)
    for t in range(1, w.n_steps + 1):
        pos = w.n_ctx + t - 1
        B.lrkv_append(L, K[:, :, pos].contiguous(), V[:, :, pos].contiguous(), pos)
        n = pos + 1
        q = np.stack([synth.queries(w, 3, t, b) for b in range(w.batch)]).astype(np.float64)
        got = run_decode(L, w, n, q)
        if t in (1, 2, w.window + 1, w.window + 2, w.n_steps) or t % 9 == 0:
            units = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
            compare_on_device_choice(got, c, units, n, q, nfit, L, f"lowram_append_W{window}_R{R}_t{t}")


def test_lowram_full_size_llama_32k_sampled():
    """The 32K Llama-3.1-8B-shaped layer (values partly predictable from keys),
    R = 4: GPU compression and fit, then one decode with 32 splits, sampled units."""
    w = LLAMA
    c = lr_case(w, 4)
    announce(f"lowram full size llama31_8b_32k: batch {w.batch} n {w.n_ctx}")
    L, _, _, nfit = prefill(c, w.n_ctx)
    got = run_decode(L, w, w.n_ctx, c.q, 32)
    assert np.all(np.isfinite(got))
    units = [(0, 0), (w.batch // 2, w.n_kv_heads // 2), (w.batch - 1, w.n_kv_heads - 1)]
    compare_on_device_choice(got, c, units, w.n_ctx, c.q, nfit, L, "lowram_full_llama31_8b_32k")
