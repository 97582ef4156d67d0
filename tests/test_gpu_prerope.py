"""Keys compressed before RoPE on the GPU (Palu: keys reconstructed on the fly)
against the oracle (oracle_decode_unit_prerope, oracle.rope).

The codes hold projections of pre-RoPE keys; the decode reconstructs each key,
rotates it to its position and scores it with the post-RoPE query; anchors are
post-RoPE keys.

  decode   oracle-made codes (bf16 of the exact projection) and oracle-rotated
           anchors: 2e-3 of max |out|, the bar of bf16 codes
  e2e      GPU prefill compression of pre-RoPE keys, post-RoPE anchors, appends
           of post-RoPE keys (the leaving key turned back on the GPU) and decode
           steps, against the oracle's cache from the pre-RoPE keys
  full     the 32K Llama-3.1-8B-shaped layer (positions up to 32767), sampled units
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import D, announce, check_decode, dev, host_case
from rank_kv_cache_lrkv_amd import binding as B, layout

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def rotated(x, positions, base):
    return oracle.bf16_round(oracle.rope(x, positions, base))


def expected(hc, base, units=None, n=None, q=None):
    w = hc.w
    g = w.group
    q = hc.q if q is None else q
    out = np.full((w.batch, w.n_q_heads, D), np.nan)
    units = units or [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    for b, h in units:
        nb = hc.lens[b] if n is None else n
        cpos, apos = oracle.code_positions(nb, w.window), oracle.anchor_positions(nb, w.window)
        ck = oracle.bf16_round(oracle.oracle_compress(hc.k[b][h][cpos], hc.u_k[h]))
        cv = oracle.bf16_round(oracle.oracle_compress(hc.v[b][h][cpos], hc.u_v[h]))
        rows = slice(h * g, (h + 1) * g)
        out[b, rows] = oracle.oracle_decode_unit_prerope(
            q[b, rows], hc.u_k[h], hc.u_v[h], ck, cv, cpos, rotated(hc.k[b][h][apos], apos, base),
            hc.v[b][h][apos], oracle.default_scale(), base)
    return out


def gpu_prerope_layer(hc, base):
    w, Wn = hc.w, hc.w.window
    cap = layout.round_cap(max(0, hc.n - 1 - Wn))
    L = B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                         window=Wn, cap=cap, rank_k=hc.rk, rank_v=hc.rv,
                         bases=dev(layout.pack_bases(hc.u_k, hc.u_v), "bf16"), rope_base=base)
    ck = np.zeros(max(1, layout.codes_elems(hc.rk, w.batch, cap)), np.float32)
    cv = np.zeros(max(1, layout.codes_elems(hc.rv, w.batch, cap)), np.float32)
    ok, ov = layout.code_offsets(hc.rk, w.batch, cap), layout.code_offsets(hc.rv, w.batch, cap)
    ak = np.zeros((w.batch, w.n_kv_heads, 1 + Wn, D), np.float32)
    av = np.zeros_like(ak)
    for b in range(w.batch):
        cpos, apos = oracle.code_positions(hc.lens[b], Wn), oracle.anchor_positions(hc.lens[b], Wn)
        for h in range(w.n_kv_heads):
            for which, flat, off, r in (("k", ck, ok, hc.rk), ("v", cv, ov, hc.rv)):
                src = (hc.k if which == "k" else hc.v)[b][h][cpos]
                u = (hc.u_k if which == "k" else hc.u_v)[h]
                codes = oracle.bf16_round(oracle.oracle_compress(src, u)).astype(np.float32)
                base_off = off[h] + b * cap * int(r[h])
                flat[base_off:base_off + cap * int(r[h])] = layout.pack_codes(codes, cap, which)
            kr = rotated(hc.k[b][h][apos], apos, base)
            for i, p in enumerate(apos):
                s = layout.anchor_slot(int(p), Wn)
                ak[b, h, s] = kr[i]
                av[b, h, s] = hc.v[b][h][p]
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


BASE = W["qwen3_1p7b_4k"].scaled(batch=2, n_q_heads=8, n_kv_heads=2, window=16)

DECODE = [
    # label, workload, rope base, n_splits, ragged lengths
    ("llama_n3000_s32", W["llama31_8b_32k"].scaled(batch=1, n_ctx=3000), 500000.0, 32, None),
    # one and three splits: 40+ blocks per wave, so the angles carried from block
    # to block are reduced from the position again along the way
    ("llama_n6000_s1", W["llama31_8b_32k"].scaled(batch=1, n_ctx=6000), 500000.0, 1, None),
    ("llama_n5000_s3_b2", W["llama31_8b_32k"].scaled(batch=2, n_ctx=5000), 500000.0, 3, None),
    ("qwen_n1000", W["qwen3_1p7b_4k"].scaled(batch=2, n_ctx=1000), 1000000.0, 0, None),
    ("hc_n777_base1e4", W["llama31_8b_hc_8k"].scaled(batch=3, n_ctx=777), 10000.0, 0, None),
    ("mixed_ranks_n2000", W["llama31_8b_32layer"].scaled(batch=2, n_ctx=2000, n_steps=0), 500000.0, 0, None),
    ("ranks_16_48_96_128", BASE.scaled(n_kv_heads=4, n_q_heads=8, n_ctx=500, mixed_ranks=True,
                                       rank_k_choices=(16, 48, 96, 128), rank_v_choices=(16, 48, 96, 128)),
     10000.0, 0, None),
    ("n1", BASE.scaled(n_ctx=1), 10000.0, 0, None),
    ("n_window_plus_2", BASE.scaled(n_ctx=18), 10000.0, 0, None),
    ("window0", BASE.scaled(window=0, n_ctx=300), 10000.0, 0, None),
    ("empty_splits", BASE.scaled(n_ctx=17 + 40), 10000.0, 16, None),
    ("many_splits", BASE.scaled(n_ctx=700), 10000.0, 300, None),
    ("gqa_g16", BASE.scaled(n_q_heads=32, n_ctx=400), 10000.0, 0, None),
    ("ragged", BASE.scaled(batch=5, n_ctx=800), 10000.0, 0, [800, 1, 17, 18, 433]),
]


@pytest.mark.parametrize("label,w,base,S,lens", DECODE, ids=[d[0] for d in DECODE])
def test_prerope_decode(label, w, base, S, lens):
    announce(f"pre-RoPE decode {label}: base {base} batch {w.batch} n {w.n_ctx} S {S}")
    hc = host_case(w, lens=lens)
    got = run_decode(gpu_prerope_layer(hc, base), w, hc.n, hc.q, S, lens)
    check_decode(got, expected(hc, base), "bf16", f"prerope_{label}")


def test_prerope_decode_peaky():
    w = BASE.scaled(n_ctx=900)
    hc = host_case(w, q_scale=8.0)
    announce("pre-RoPE decode peaky q x8")
    check_decode(run_decode(gpu_prerope_layer(hc, 10000.0), w, hc.n, hc.q), expected(hc, 10000.0), "bf16",
                 "prerope_peaky")


def rows_tensor(hc, which, n, base=None):
    """[batch][Hkv][n][128]: the rows as stored, rotated to their positions if base is given."""
    src = hc.k if which == "k" else hc.v
    a = np.stack([np.stack([(rotated(src[b][h][:n], np.arange(n), base) if base else src[b][h][:n])
                            for h in range(hc.w.n_kv_heads)]) for b in range(hc.w.batch)])
    return dev(a, "bf16")


def prefill(hc, base, n, extra=0):
    w = hc.w
    c = max(0, n - 1 - w.window)
    L = B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                         window=w.window, cap=layout.round_cap(c + extra), rank_k=hc.rk, rank_v=hc.rv,
                         bases=dev(layout.pack_bases(hc.u_k, hc.u_v), "bf16"), rope_base=base)
    K_pre, V = rows_tensor(hc, "k", w.n_total), rows_tensor(hc, "v", w.n_total)
    K_rot = rows_tensor(hc, "k", w.n_total, base)
    B.lrkv_compress(L, 0, K_pre[:, :, 1:], c, 0)
    B.lrkv_compress(L, 1, V[:, :, 1:], c, 0)
    B.lrkv_store_anchors(L, K_rot[:, :, 0:1], V[:, :, 0:1], 0, 1)
    lo = max(1, n - w.window)
    B.lrkv_store_anchors(L, K_rot[:, :, lo:n], V[:, :, lo:n], lo, n - lo)
    return L, K_rot, V


@pytest.mark.parametrize("window", [0, 1, 16])
def test_prerope_decode_steps_with_append(window):
    w = W["llama31_8b_32k"].scaled(batch=2, n_ctx=60, n_steps=40, window=window)
    base = 500000.0
    announce(f"pre-RoPE e2e append steps W={window}")
    hc = host_case(w, layer=3)
    hc.lens = [w.n_total] * w.batch
    L, K_rot, V = prefill(hc, base, w.n_ctx, extra=w.n_steps)
    for t in range(1, w.n_steps + 1):
        pos = w.n_ctx + t - 1
        B.lrkv_append(L, K_rot[:, :, pos].contiguous(), V[:, :, pos].contiguous(), pos)
        n = pos + 1
        q = np.stack([synth.queries(w, 3, t, b) for b in range(w.batch)]).astype(np.float64)
        got = run_decode(L, w, n, q)
        if t in (1, 2, w.window + 1, w.window + 2, w.n_steps) or t % 9 == 0:
            check_decode(got, expected(hc, base, n=n, q=q), "bf16", f"prerope_append_W{window}_t{t}")


def test_prerope_full_size_llama_32k_sampled():
    """The 32K Llama-3.1-8B-shaped layer (RoPE base 500000, positions up to
    32767), 32 splits: GPU prefill compression of the pre-RoPE keys, one decode,
    sampled units."""
    w = W["llama31_8b_32k"]
    base = 500000.0
    hc = host_case(w)
    announce(f"pre-RoPE full size llama31_8b_32k: batch {w.batch} n {w.n_ctx}")
    L, _, _ = prefill(hc, base, w.n_ctx)
    got = run_decode(L, w, w.n_ctx, hc.q, 32)
    assert np.all(np.isfinite(got))
    units = [(0, 0), (w.batch // 2, w.n_kv_heads // 2), (w.batch - 1, w.n_kv_heads - 1)]
    check_decode(got, expected(hc, base, units), "bf16", "prerope_full_llama31_8b_32k")


@pytest.mark.parametrize("base,S", [(500000.0, 2), (10000.0, 3)])
def test_prerope_long_positions(base, S):
    """Positions up to 131,071 on one KV head with two or three splits: each wave
    carries its pair angles over ~500 blocks at a stride of 8 or 12 blocks,
    reducing them from the position again every 16 blocks."""
    w = W["llama31_8b_32k"].scaled(batch=1, n_q_heads=4, n_kv_heads=1, n_ctx=131072)
    hc = host_case(w)
    announce(f"pre-RoPE long positions: base {base} n {w.n_ctx} S {S}")
    L = gpu_prerope_layer(hc, base)
    got = run_decode(L, w, w.n_ctx, hc.q, S)
    check_decode(got, expected(hc, base), "bf16", f"prerope_long_{int(base)}_s{S}")
