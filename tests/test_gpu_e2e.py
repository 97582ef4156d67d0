"""End to end on the GPU: prefill compression, anchor stores, decode steps with
cache maintenance, against the oracle (which makes its own codes from the same
keys and values).  Includes the five workloads at their full sizes, checked on
sampled (batch row, KV head) units the oracle computes one by one."""

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import D, announce, check_decode, dev, host_case, gpu_layer, to_storage
from rank_kv_cache_lrkv_amd import binding as B, layout

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def full_rows(w, layer, which):
    """[batch][Hkv][n_total][128] float32 storage values, generated unit by unit."""
    a = np.empty((w.batch, w.n_kv_heads, w.n_total, D), np.float32)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            a[b, h] = synth.unit_kv(w, layer, h, b, which)
    return a


def bases_flat(w, layer):
    rk, rv = synth.ranks(w, layer)
    return rk, rv, layout.pack_bases([synth.basis(w, layer, h, "k", int(rk[h])) for h in range(w.n_kv_heads)],
                                     [synth.basis(w, layer, h, "v", int(rv[h])) for h in range(w.n_kv_heads)])


def prefill(w, layer, n, cap=None):
    """Allocate a layer, compress tokens 1..n-W-1 and store the anchors of a
    context of n tokens, all on the GPU.  Returns (Layer, K, V) (K, V on GPU)."""
    rk, rv, bases = bases_flat(w, layer)
    cmax = max(0, n - 1 - w.window)
    cap = layout.round_cap(cmax + w.n_steps) if cap is None else cap
    L = B.Layer.allocate(dtype=B.LRKV_F32 if w.dtype == "f32" else B.LRKV_BF16, batch=w.batch,
                         n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads, window=w.window, cap=cap,
                         rank_k=rk, rank_v=rv, bases=dev(bases, w.dtype))
    K = dev(full_rows(w, layer, "k"), w.dtype)
    V = dev(full_rows(w, layer, "v"), w.dtype)
    B.lrkv_compress(L, 0, K[:, :, 1:], cmax, 0)
    B.lrkv_compress(L, 1, V[:, :, 1:], cmax, 0)
    B.lrkv_store_anchors(L, K[:, :, 0:1], V[:, :, 0:1], 0, 1)
    lo = max(1, n - w.window)
    B.lrkv_store_anchors(L, K[:, :, lo:n], V[:, :, lo:n], lo, n - lo)
    return L, K, V


def oracle_units(w, layer, n, step, units, q):
    """Oracle output for the listed (b, h) units at context n (float64)."""
    rk, rv = synth.ranks(w, layer)
    g = w.group
    out = np.full((w.batch, w.n_q_heads, D), np.nan)
    cpos, apos = oracle.code_positions(n, w.window), oracle.anchor_positions(n, w.window)
    for b, h in units:
        k = synth.unit_kv(w, layer, h, b, "k").astype(np.float64)
        v = synth.unit_kv(w, layer, h, b, "v").astype(np.float64)
        uk = synth.basis(w, layer, h, "k", int(rk[h])).astype(np.float64)
        uv = synth.basis(w, layer, h, "v", int(rv[h])).astype(np.float64)
        ck = to_storage(oracle.oracle_compress(k[cpos], uk), w.dtype)
        cv = to_storage(oracle.oracle_compress(v[cpos], uv), w.dtype)
        rows = slice(h * g, (h + 1) * g)
        out[b, rows] = oracle.oracle_decode_unit(q[b, rows], uk, uv, ck, cv, k[apos], v[apos],
                                                 oracle.default_scale())
    return out


def decode(L, w, n, q_np, S):
    q = dev(q_np, w.dtype)
    out = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device="cuda")
    ws = B.workspace(L, S)
    B.lrkv_decode_attn(L, n, q, out, oracle.default_scale(), S, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def queries(w, layer, step):
    return np.stack([synth.queries(w, layer, step, b) for b in range(w.batch)]).astype(np.float64)


def sample_units(w, k=3):
    us = {(0, 0), (w.batch - 1, w.n_kv_heads - 1), (w.batch // 2, w.n_kv_heads // 2)}
    return sorted(us)[:k]


REDUCED = [
    ("tiny_f32", W["tiny_f32"]),
    ("qwen3_n1500", W["qwen3_1p7b_4k"].scaled(batch=2, n_ctx=1500)),
    ("hc_n600", W["llama31_8b_hc_8k"].scaled(batch=2, n_ctx=600)),
]


@pytest.mark.parametrize("label,w", REDUCED, ids=[r[0] for r in REDUCED])
def test_prefill_then_decode(label, w):
    announce(f"e2e prefill+decode {label}")
    L, _, _ = prefill(w, 0, w.n_ctx)
    q = queries(w, 0, 0)
    S = B.lrkv_decode_auto_splits(L, w.n_ctx)
    got = decode(L, w, w.n_ctx, q, S)
    units = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    check_decode(got, oracle_units(w, 0, w.n_ctx, 0, units, q), w.dtype, f"e2e_{label}")


@pytest.mark.parametrize("window", [0, 1, 16])
def test_decode_steps_with_append(window):
    """The decode loop: append the new token (compressing the one that leaves the
    window), then decode; every step against the oracle from scratch."""
    w = W["llama31_8b_32layer"].scaled(batch=2, n_ctx=60, n_steps=40, window=window)
    announce(f"e2e append steps W={window}")
    L, K, V = prefill(w, 3, w.n_ctx)
    units = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    for t in range(1, w.n_steps + 1):
        pos = w.n_ctx + t - 1
        B.lrkv_append(L, K[:, :, pos].contiguous(), V[:, :, pos].contiguous(), pos)
        n = pos + 1
        q = queries(w, 3, t)
        got = decode(L, w, n, q, B.lrkv_decode_auto_splits(L, n))
        if t in (1, 2, w.window + 1, w.window + 2, w.n_steps) or t % 9 == 0:
            check_decode(got, oracle_units(w, 3, n, t, units, q), "bf16", f"append_W{window}_t{t}")


def test_append_from_empty_cache():
    """Build the cache token by token from position 0 with append only."""
    w = W["qwen3_1p7b_4k"].scaled(batch=1, n_q_heads=4, n_kv_heads=2, window=4, n_ctx=0, n_steps=40)
    rk, rv, bases = bases_flat(w, 0)
    L = B.Layer.allocate(dtype=B.LRKV_BF16, batch=1, n_q_heads=4, n_kv_heads=2, window=4, cap=64,
                         rank_k=rk, rank_v=rv, bases=dev(bases, "bf16"))
    K = dev(full_rows(w, 0, "k"), "bf16")
    V = dev(full_rows(w, 0, "v"), "bf16")
    announce("e2e append from empty")
    units = [(0, 0), (0, 1)]
    for pos in range(40):
        B.lrkv_append(L, K[:, :, pos].contiguous(), V[:, :, pos].contiguous(), pos)
        n = pos + 1
        if n in (1, 2, 5, 6, 7, 40):
            q = queries(w, 0, n)
            check_decode(decode(L, w, n, q, 2), oracle_units(w, 0, n, n, units, q), "bf16", f"from_empty_n{n}")


# ---------------------------------------------------------------------------
# full sizes, sampled units
# ---------------------------------------------------------------------------

FULL = [("qwen3_1p7b_4k", 0), ("llama31_8b_32k", 32), ("llama31_8b_hc_8k", 0), ("tiny_f32", 0)]


@pytest.mark.parametrize("name,S", FULL, ids=[f[0] for f in FULL])
def test_full_size_sampled(name, S):
    w = W[name]
    announce(f"full size {name}: batch {w.batch} n {w.n_ctx}")
    L, _, _ = prefill(w, 0, w.n_ctx)
    S = S or B.lrkv_decode_auto_splits(L, w.n_ctx)
    q = queries(w, 0, 0)
    got = decode(L, w, w.n_ctx, q, S)
    assert np.all(np.isfinite(got))
    check_decode(got, oracle_units(w, 0, w.n_ctx, 0, sample_units(w), q), w.dtype, f"full_{name}")


def prefill_rows(w, layer, n, kv):
    """As ``prefill`` from already generated host rows kv = {"k": .., "v": ..}."""
    rk, rv, bases = bases_flat(w, layer)
    cmax = max(0, n - 1 - w.window)
    L = B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                         window=w.window, cap=layout.round_cap(cmax + w.n_steps), rank_k=rk, rank_v=rv,
                         bases=dev(bases, w.dtype))
    K, V = dev(kv["k"], w.dtype), dev(kv["v"], w.dtype)
    B.lrkv_compress(L, 0, K[:, :, 1:], cmax, 0)
    B.lrkv_compress(L, 1, V[:, :, 1:], cmax, 0)
    B.lrkv_store_anchors(L, K[:, :, 0:1], V[:, :, 0:1], 0, 1)
    lo = max(1, n - w.window)
    B.lrkv_store_anchors(L, K[:, :, lo:n], V[:, :, lo:n], lo, n - lo)
    return L, K, V


def step_units(w, t):
    """Units compared at decode step t (1-based): two per step, rotating so that
    over the steps every (batch row, KV head) unit of the layer is compared at
    least once, and every unit at the last step."""
    units = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    if t == w.n_steps:
        return units
    k = len(units)
    return [units[(2 * (t - 1)) % k], units[(2 * (t - 1) + 1) % k]]


@pytest.mark.parametrize("layer", range(32))
def test_full_size_32layer_decode_steps(layer):
    """32-layer workload at full context, every layer: prefill 32768 tokens with the
    layer's mixed ranks, then 16 decode steps with cache maintenance; at each step
    the decode output of two (batch row, KV head) units (rotating over the layer's
    32 units) is compared with the oracle, and all 32 units at the last step."""
    w = W["llama31_8b_32layer"]
    rk, rv = synth.ranks(w, layer)
    announce(f"full 32-layer workload, layer {layer}, ranks {rk.tolist()} / {rv.tolist()}")
    kv = {x: full_rows(w, layer, x) for x in "kv"}
    L, K, V = prefill_rows(w, layer, w.n_ctx, kv)
    # oracle side: the exact projection of every code row up to the last step's
    # context, once per unit (each code row is its own x U; a context's codes are
    # the first rows), rounded to bf16 as stored
    n_last = w.n_total
    cpos_last = oracle.code_positions(n_last, w.window)
    uk = [synth.basis(w, layer, h, "k", int(rk[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    uv = [synth.basis(w, layer, h, "v", int(rv[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    codes = {}

    def unit_codes(b, h):
        if (b, h) not in codes:
            k = kv["k"][b, h].astype(np.float64)
            v = kv["v"][b, h].astype(np.float64)
            codes[(b, h)] = (to_storage(oracle.oracle_compress(k[cpos_last], uk[h]), w.dtype),
                             to_storage(oracle.oracle_compress(v[cpos_last], uv[h]), w.dtype))
        return codes[(b, h)]

    g = w.group
    compared = set()
    for t in range(1, w.n_steps + 1):
        pos = w.n_ctx + t - 1
        B.lrkv_append(L, K[:, :, pos].contiguous(), V[:, :, pos].contiguous(), pos)
        n = pos + 1
        q = queries(w, layer, t)
        got = decode(L, w, n, q, B.lrkv_decode_auto_splits(L, n))
        assert np.all(np.isfinite(got))
        nc = len(oracle.code_positions(n, w.window))
        apos = oracle.anchor_positions(n, w.window)
        want = np.full_like(got, np.nan)
        for b, h in step_units(w, t):
            ck, cv = unit_codes(b, h)
            rows = slice(h * g, (h + 1) * g)
            want[b, rows] = oracle.oracle_decode_unit(
                q[b, rows], uk[h], uv[h], ck[:nc], cv[:nc], kv["k"][b, h][apos].astype(np.float64),
                kv["v"][b, h][apos].astype(np.float64), oracle.default_scale())
            compared.add((b, h))
        check_decode(got, want, "bf16", f"l{layer}_step{t}")
    assert len(compared) == w.batch * w.n_kv_heads
