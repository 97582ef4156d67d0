"""Decode over codes made under several basis versions (OjaKV: the basis keeps
adapting, older codes keep the basis they were made with) against the oracle's
oracle_decode_unit_versions, and the OjaKV decode loop end to end: prefill,
decode steps with appends, an Oja update that opens a new version, more steps.
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import D, announce, check_decode, code_storage, oracle_quant
from rank_kv_cache_lrkv_amd import binding as B, layout

pytestmark = pytest.mark.gpu


def bf16t(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def basis(rng, r):
    q, _ = np.linalg.qr(rng.standard_normal((D, D)))
    return oracle.bf16_round(q[:, :r])


def kv_rows(rng, n):
    sig = np.exp(-np.arange(D) / 16.0)
    q, _ = np.linalg.qr(rng.standard_normal((D, D)))
    return oracle.bf16_round((rng.standard_normal((n, D)) * sig) @ q.T)


def slot_versions(starts, c):
    """Version of code slots 0 .. c-1: the last version starting at or before it."""
    j = np.arange(c)
    return np.searchsorted(np.asarray(starts), j, side="right") - 1


def build(rng, batch, n_kv, g, lens, W, rk, rv, starts, qbits=0):
    """A versioned layer on the GPU with oracle-made codes, and the oracle's output."""
    V = len(starts[0])
    bk = [[basis(rng, rk) for _ in range(n_kv)] for _ in range(V)]
    bv = [[basis(rng, rv) for _ in range(n_kv)] for _ in range(V)]
    n_max = max(lens)
    k = [[kv_rows(rng, n_max) for _ in range(n_kv)] for _ in range(batch)]
    v = [[kv_rows(rng, n_max) for _ in range(n_kv)] for _ in range(batch)]
    q = oracle.bf16_round(rng.standard_normal((batch, n_kv * g, D)))
    cap = layout.round_cap(max(1, n_max - 1 - W))
    dtype = {0: B.LRKV_BF16, 8: B.LRKV_BF16_Q8, 4: B.LRKV_BF16_Q4}[qbits]
    flat = np.concatenate([layout.pack_bases(bk[ver], bv[ver]) for ver in range(V)])
    L = B.Layer.allocate(dtype=dtype, batch=batch, n_q_heads=n_kv * g, n_kv_heads=n_kv, window=W, cap=cap,
                         rank_k=[rk] * n_kv, rank_v=[rv] * n_kv, bases=bf16t(flat).cuda(), n_versions=V)
    L.version_start.copy_(torch.tensor(starts, dtype=torch.int32))
    kind = f"q{qbits}" if qbits else "bf16"
    ck = np.zeros(layout.codes_elems([rk] * n_kv, batch, cap), np.int8 if qbits else np.float32)
    cv = np.zeros(layout.codes_elems([rv] * n_kv, batch, cap), np.int8 if qbits else np.float32)
    sk = np.zeros(layout.scales_elems(n_kv, batch, cap) if qbits else 1, np.float32)
    sv = np.zeros_like(sk)
    ak = np.zeros((batch, n_kv, 1 + W, D), np.float32)
    av = np.zeros_like(ak)
    want = np.full((batch, n_kv * g, D), np.nan)
    for b in range(batch):
        n = lens[b]
        cpos, apos = oracle.code_positions(n, W), oracle.anchor_positions(n, W)
        ver = slot_versions(starts[b], len(cpos))
        for h in range(n_kv):
            codes = {}
            for which, src, bases, flatc, sc, r in (("k", k, bk, ck, sk, rk), ("v", v, bv, cv, sv, rv)):
                exact = np.stack([src[b][h][p] @ bases[vj][h] for p, vj in zip(cpos, ver)]) \
                    if len(cpos) else np.zeros((0, r))
                base = h * batch * cap * r + b * cap * r
                if qbits:
                    qq, ss = oracle_quant(exact, qbits)
                    flatc[base:base + cap * r] = layout.pack_codes(qq, cap, which)
                    s0 = layout.scale_offset(h, b, cap, batch)
                    sc[s0:s0 + len(ss)] = ss
                else:
                    flatc[base:base + cap * r] = layout.pack_codes(
                        oracle.bf16_round(exact).astype(np.float32), cap, which)
                codes[which] = code_storage(exact, kind)
            for p in apos:
                ak[b, h, layout.anchor_slot(int(p), W)] = k[b][h][p]
                av[b, h, layout.anchor_slot(int(p), W)] = v[b][h][p]
            rows = slice(h * g, (h + 1) * g)
            want[b, rows] = oracle.oracle_decode_unit_versions(
                q[b, rows], [bk[x][h] for x in range(V)], [bv[x][h] for x in range(V)], ver,
                codes["k"], codes["v"], k[b][h][apos], v[b][h][apos], oracle.default_scale())
    if qbits:
        if qbits == 4:
            ck, cv = layout.pack_nibbles(ck), layout.pack_nibbles(cv)
        L.codes_k.copy_(torch.from_numpy(ck).cuda())
        L.codes_v.copy_(torch.from_numpy(cv).cuda())
        L.scales_k.copy_(torch.from_numpy(sk).cuda())
        L.scales_v.copy_(torch.from_numpy(sv).cuda())
    else:
        L.codes_k.copy_(bf16t(ck).cuda())
        L.codes_v.copy_(bf16t(cv).cuda())
    L.anchor_k.copy_(bf16t(ak).cuda())
    L.anchor_v.copy_(bf16t(av).cuda())
    return L, bf16t(q).cuda(), want


def run(L, q, n, lens, S):
    out = torch.empty((L.batch, L.n_q_heads, D), dtype=torch.float32, device="cuda")
    ws = B.workspace(L, S)
    cl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    B.lrkv_decode_attn(L, n, q, out, oracle.default_scale(), S, ws, ctx_lens=cl)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


CASES = [
    # label, batch, lens, W, starts per row, splits
    ("two_versions", 2, [900, 700], 16, [[0, 320], [0, 96]], 0),
    ("three_versions_min_splits", 2, [1200, 1000], 16, [[0, 320, 640], [0, 32, 800]], 3),
    ("empty_middle_version", 2, [700, 300], 8, [[0, 192, 192], [0, 64, 64]], 0),
    ("version_past_context", 1, [500], 16, [[0, 4096]], 0),
    ("many_splits", 1, [2000], 64, [[0, 960, 1600]], 200),
    ("ragged_short_rows", 3, [800, 20, 1], 16, [[0, 256], [0, 32], [0, 32]], 0),
]


@pytest.mark.parametrize("label,batch,lens,W,starts,S", CASES, ids=[c[0] for c in CASES])
def test_versioned_decode(label, batch, lens, W, starts, S):
    rng = np.random.default_rng(sum(map(ord, label)))
    L, q, want = build(rng, batch, 2, 4, lens, W, 64, 32, starts)
    S = S or B.lrkv_decode_auto_splits(L, max(lens))
    announce(f"versioned decode {label}: V {len(starts[0])} S {S} lens {lens}")
    check_decode(run(L, q, max(lens), lens, S), want, "bf16", f"versions_{label}")


@pytest.mark.parametrize("qbits", [8, 4])
def test_versioned_decode_quantised(qbits):
    rng = np.random.default_rng(50 + qbits)
    lens = [1000, 640]
    L, q, want = build(rng, 2, 2, 4, lens, 16, 64, 32, [[0, 416], [0, 160]], qbits=qbits)
    announce(f"versioned decode, {qbits}-bit codes")
    check_decode(run(L, q, 1000, lens, B.lrkv_decode_auto_splits(L, 1000)), want, "bf16", f"versions_q{qbits}")


def test_oja_decode_loop_end_to_end():
    """Prefill with the calibration basis, Oja steps over the prompt (in place),
    compress the prompt with the adapted basis; decode steps with appends; then
    an Oja step over the tokens that left the window opens version 1 at the next
    32-slot boundary, and the steps go on.  Every checked step is compared with
    the oracle rebuilt from scratch: its bases are its own chain of Oja steps from
    the same rows, each rounded to bf16 as the device stores it, so the two sides'
    bases may differ by one bf16 step in a few entries (the update's own parity is
    in test_gpu_oja.py)."""
    w = synth.WORKLOADS["llama31_8b_32layer"].scaled(batch=2, n_ctx=400, n_steps=120, window=16)
    layer = 1
    rk, rv = synth.ranks(w, layer)
    K = np.stack([np.stack([synth.unit_kv(w, layer, h, b, "k") for h in range(w.n_kv_heads)])
                  for b in range(w.batch)])
    V_ = np.stack([np.stack([synth.unit_kv(w, layer, h, b, "v") for h in range(w.n_kv_heads)])
                   for b in range(w.batch)])
    Kd, Vd = bf16t(K).cuda(), bf16t(V_).cuda()
    bases0 = layout.pack_bases([synth.basis(w, layer, h, "k", int(rk[h])) for h in range(w.n_kv_heads)],
                               [synth.basis(w, layer, h, "v", int(rv[h])) for h in range(w.n_kv_heads)])
    nb = bases0.size
    cap = layout.round_cap(w.n_ctx + w.n_steps)
    L = B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                         window=w.window, cap=cap, rank_k=rk, rank_v=rv, n_versions=2,
                         bases=torch.cat([bf16t(bases0), torch.zeros(nb, dtype=torch.bfloat16)]).cuda())
    L.version_start.fill_(1 << 30)                    # version 1 not open yet
    L.version_start[:, 0] = 0
    n = w.n_ctx
    c = n - 1 - w.window
    announce("oja loop: adapt on the prompt, compress, decode, adapt again")
    for _ in range(2):                                # adapt version 0 in place on the prompt's rows
        B.lrkv_oja_update(L, 0, Kd[:, :, 1:], n - 1, 0.5, 0, 0)
        B.lrkv_oja_update(L, 1, Vd[:, :, 1:], n - 1, 0.5, 0, 0)
    # compress with the latest version: version 1 must equal version 0 for now
    L.bases[nb:] = L.bases[:nb]
    B.lrkv_compress(L, 0, Kd[:, :, 1:], c, 0)
    B.lrkv_compress(L, 1, Vd[:, :, 1:], c, 0)
    B.lrkv_store_anchors(L, Kd[:, :, 0:1], Vd[:, :, 0:1], 0, 1)
    B.lrkv_store_anchors(L, Kd[:, :, n - w.window:n], Vd[:, :, n - w.window:n], n - w.window, w.window)
    torch.cuda.synchronize()
    starts = np.array([[0, 1 << 30]] * w.batch)
    # the oracle's bases: the same steps from the same bf16 rows and basis
    ob_k = [synth.basis(w, layer, h, "k", int(rk[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    ob_v = [synth.basis(w, layer, h, "v", int(rv[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    rows_k = [K[:, h, 1:n].reshape(-1, D).astype(np.float64) for h in range(w.n_kv_heads)]
    rows_v = [V_[:, h, 1:n].reshape(-1, D).astype(np.float64) for h in range(w.n_kv_heads)]
    for _ in range(2):
        ob_k = [oracle.bf16_round(oracle.oja_update(u, x, 0.5)) for u, x in zip(ob_k, rows_k)]
        ob_v = [oracle.bf16_round(oracle.oja_update(u, x, 0.5)) for u, x in zip(ob_v, rows_v)]
    obases = [[ob_k, ob_v], [ob_k, ob_v]]             # versions 0 and 1 (1 = 0 until opened)
    opened = None
    for t in range(1, w.n_steps + 1):
        pos = n + t - 1
        if t == 60:  # adapt on the last 59 tokens that left the window, open version 1
            lo = pos - w.window - 59
            B.lrkv_oja_update(L, 0, Kd[:, :, lo:pos - w.window], 59, 0.5, 0, 1)
            B.lrkv_oja_update(L, 1, Vd[:, :, lo:pos - w.window], 59, 0.5, 0, 1)
            ek = [K[:, h, lo:pos - w.window].reshape(-1, D).astype(np.float64) for h in range(w.n_kv_heads)]
            ev = [V_[:, h, lo:pos - w.window].reshape(-1, D).astype(np.float64) for h in range(w.n_kv_heads)]
            obases[1] = [[oracle.bf16_round(oracle.oja_update(u, x, 0.5)) for u, x in zip(ob_k, ek)],
                         [oracle.bf16_round(oracle.oja_update(u, x, 0.5)) for u, x in zip(ob_v, ev)]]
            slot = pos - w.window - 1
            opened = (slot + 31) // 32 * 32
            starts[:, 1] = opened
            L.version_start.copy_(torch.tensor(starts, dtype=torch.int32))
        B.lrkv_append(L, Kd[:, :, pos].contiguous(), Vd[:, :, pos].contiguous(), pos)
        if t in (1, 59, 60, 61, 90, w.n_steps):
            nn = pos + 1
            qn = np.stack([synth.queries(w, layer, t, b) for b in range(w.batch)]).astype(np.float64)
            out = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device="cuda")
            S = B.lrkv_decode_auto_splits(L, nn)
            B.lrkv_decode_attn(L, nn, bf16t(qn).cuda(), out, oracle.default_scale(), S, B.workspace(L, S))
            torch.cuda.synchronize()
            want = np.empty((w.batch, w.n_q_heads, D))
            cpos, apos = oracle.code_positions(nn, w.window), oracle.anchor_positions(nn, w.window)
            ver = slot_versions(starts[0], len(cpos))
            g = w.group
            for b in range(w.batch):
                for h in range(w.n_kv_heads):
                    bk = [obases[x][0][h] for x in range(2)]
                    bv = [obases[x][1][h] for x in range(2)]
                    kk, vv = K[b, h].astype(np.float64), V_[b, h].astype(np.float64)
                    ck = oracle.bf16_round(np.stack([kk[p] @ bk[vj] for p, vj in zip(cpos, ver)]))
                    cv = oracle.bf16_round(np.stack([vv[p] @ bv[vj] for p, vj in zip(cpos, ver)]))
                    rows = slice(h * g, (h + 1) * g)
                    want[b, rows] = oracle.oracle_decode_unit_versions(
                        qn[b, rows], bk, bv, ver, ck, cv, kk[apos], vv[apos], oracle.default_scale())
            check_decode(out.cpu().numpy().astype(np.float64), want, "bf16", f"oja_loop_t{t}")
    assert opened is not None
