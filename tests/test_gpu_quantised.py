"""Quantised codes with per-token float32 scales on the GPU, int8
(LRKV_BF16_Q8) and 4-bit (LRKV_BF16_Q4), against the oracle's quantisers and
decode.

  quantise   lrkv_quantize on given float32 rows: codes and scales bit-exact
  compress   lrkv_compress from bf16 rows: every code within one step of the
             oracle's quantisation of the exact projection, scales within the
             float32 accumulation bound, >= 99.9% of codes identical
  decode     oracle-made quantised codes (so decode is checked apart from compress),
             2e-3 of max |out|, the bar of bf16 codes
  end to end prefill compression, anchors, appends and decode steps against the
             oracle's own quantised cache
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import (D, announce, check_decode, code_storage, dev, gpu_decode, gpu_layer, host_case,
                   oracle_quant)
from rank_kv_cache_lrkv_amd import binding as B, layout

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS
BITS = [8, 4]
DTYPE = {8: B.LRKV_BF16_Q8, 4: B.LRKV_BF16_Q4}
QMAX = {8: 127, 4: 7}
QUANTISE = {8: oracle.quantize_codes_q8, 4: oracle.quantize_codes_q4}


def q_layer(bits, batch, n_kv, rk, rv, cap, window=4, group=2):
    return B.Layer.allocate(dtype=DTYPE[bits], batch=batch, n_q_heads=group * n_kv, n_kv_heads=n_kv,
                            window=window, cap=cap, rank_k=rk, rank_v=rv)


def bits_of(L):
    return 4 if L.dtype == B.LRKV_BF16_Q4 else 8


def read_q(L, which, b, h, n, slot0=0):
    """(codes int8 (n, r), scales float32 (n,)) of slots slot0 .. slot0 + n - 1."""
    ranks = L.rank_k if which == "k" else L.rank_v
    r = int(ranks[h])
    off = layout.code_offsets(ranks, L.batch, L.cap)[h] + b * L.cap * r
    buf = L.codes_k if which == "k" else L.codes_v
    if bits_of(L) == 4:
        flat = layout.unpack_nibbles(buf[off // 2:(off + L.cap * r) // 2].cpu().numpy())
    else:
        flat = buf[off:off + L.cap * r].cpu().numpy()
    codes = layout.unpack_codes(flat, slot0 + n, r, which)[slot0:]
    s0 = layout.scale_offset(h, b, L.cap, L.batch)
    sc = (L.scales_k if which == "k" else L.scales_v)[s0 + slot0:s0 + slot0 + n].cpu().numpy()
    return codes, sc


# ---------------------------------------------------------------------------
# quantiser: bit-exact
# ---------------------------------------------------------------------------

def special_rows(r, rng, qmax):
    """Rows that exercise the rounding rule: ties at every half step, a zero row,
    a single nonzero, both signs of the extreme, tiny and huge magnitudes."""
    rows = []
    t = np.zeros(r, np.float32)
    t[0] = qmax
    t[1:] = (np.arange(1, r) % (2 * qmax + 1) - qmax + 0.5).astype(np.float32)  # x / s on .5: ties to even
    t = np.clip(t, -qmax, qmax)
    rows.append(t)
    rows.append(np.zeros(r, np.float32))
    one = np.zeros(r, np.float32)
    one[r // 2] = -3.0e-3
    rows.append(one)
    ext = rng.standard_normal(r).astype(np.float32)
    ext[0], ext[-1] = 5.0, -5.0
    rows.append(ext)
    rows.append((rng.standard_normal(r) * 1e-30).astype(np.float32))
    rows.append((rng.standard_normal(r) * 1e30).astype(np.float32))
    return np.stack(rows)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("which", [0, 1])
def test_quantize_bit_exact(which, bits):
    rk, rv = [16, 48, 128], [32, 16, 96]
    batch, n_kv, cap = 2, 3, 160
    L = q_layer(bits, batch, n_kv, rk, rv, cap)
    ranks = rk if which == 0 else rv
    rng = np.random.default_rng(1234 + which)
    n_tok, slot0 = 77, 5
    # rows padded to 136 floats, heads and rows strided: [batch][n_kv][n_tok][136]
    x = (rng.standard_normal((batch, n_kv, n_tok, 136)) * rng.uniform(0.01, 50, (batch, n_kv, n_tok, 1)))
    x = x.astype(np.float32)
    for b in range(batch):
        for h in range(n_kv):
            sp = special_rows(ranks[h], rng, QMAX[bits])
            x[b, h, 10:10 + len(sp), :ranks[h]] = sp
    canary = 99 if bits == 8 else -8      # 4 bits: 0x88 in every byte, a value the quantiser never makes
    (L.codes_k if which == 0 else L.codes_v).fill_(99 if bits == 8 else 0x88)
    (L.scales_k if which == 0 else L.scales_v).fill_(-1.0)
    announce(f"quantize {bits} bits which={which} ranks {ranks} n_tok {n_tok} slot0 {slot0}")
    B.lrkv_quantize(L, which, torch.from_numpy(x).cuda(), n_tok, slot0)
    torch.cuda.synchronize()
    name = "k" if which == 0 else "v"
    for b in range(batch):
        for h in range(n_kv):
            q_want, s_want = QUANTISE[bits](x[b, h, :, :ranks[h]])
            q_got, s_got = read_q(L, name, b, h, n_tok, slot0)
            assert np.array_equal(s_got.view(np.uint32), s_want.view(np.uint32)), (b, h)
            assert np.array_equal(q_got, q_want), (b, h, np.argwhere(q_got != q_want)[:5])
            allq, alls = read_q(L, name, b, h, cap)
            assert np.all(allq[:slot0] == canary) and np.all(allq[slot0 + n_tok:] == canary)
            assert np.all(alls[:slot0] == -1.0) and np.all(alls[slot0 + n_tok:] == -1.0)


def test_quantize_hand_examples():
    """The oracle pins' hand-worked rows, through the GPU quantisers."""
    L = q_layer(8, 1, 1, [16], [16], 32)
    x = np.zeros((1, 1, 2, 16), np.float32)
    x[0, 0, 0, :5] = [127, -63.5, 0.25, 0, 62.5]
    x[0, 0, 1, :5] = [254, 1, -3, 5, -254]
    announce("quantize hand examples")
    B.lrkv_quantize(L, 0, torch.from_numpy(x).cuda(), 2, 0)
    torch.cuda.synchronize()
    q, s = read_q(L, "k", 0, 0, 2)
    assert s.tolist() == [1.0, 2.0]
    assert q[0, :5].tolist() == [127, -64, 0, 0, 62]
    assert q[1, :5].tolist() == [127, 0, -2, 2, -127]
    assert np.all(q[:, 5:] == 0)
    L4 = q_layer(4, 1, 1, [16], [16], 32)
    x4 = np.zeros((1, 1, 2, 16), np.float32)
    x4[0, 0, 0, :5] = [7, -3.5, 0.25, 0, 2.5]
    x4[0, 0, 1, :5] = [14, 1, -3, 5, -14]
    B.lrkv_quantize(L4, 1, torch.from_numpy(x4).cuda(), 2, 0)
    torch.cuda.synchronize()
    q, s = read_q(L4, "v", 0, 0, 2)
    assert s.tolist() == [1.0, 2.0]
    assert q[0, :5].tolist() == [7, -4, 0, 0, 2]
    assert q[1, :5].tolist() == [7, 0, -2, 2, -7]
    assert np.all(q[:, 5:] == 0)


# ---------------------------------------------------------------------------
# compress from bf16 rows
# ---------------------------------------------------------------------------

def check_q_codes(q_got, s_got, x, u, bits, label):
    exact = oracle.oracle_compress(x, u)
    q_want, s_want = oracle_quant(exact, bits)
    if not q_got.size:
        return
    # float32 accumulation bound of each code, then of the row maximum
    uu = 2.0 ** -24
    gamma = D * uu / (1 - D * uu)
    acc = gamma * (np.abs(x) @ np.abs(u))
    s_tol = np.max(acc, axis=1) / QMAX[bits] + 2 * np.spacing(s_want.astype(np.float32)).astype(np.float64)
    s_err = np.abs(s_got.astype(np.float64) - s_want)
    assert np.all(s_err <= s_tol), (label, float(np.max(s_err / s_tol)))
    dq = np.abs(q_got.astype(np.int32) - q_want.astype(np.int32))
    equal = float(np.mean(dq == 0))
    print(f"[parity] {label}: {bits}-bit codes equal {equal:.5f}, max |dq| {int(dq.max())}", flush=True)
    assert dq.max() <= 1, label
    assert equal >= 0.999, (label, equal)


CASES = [
    ("qwen3_n1000", W["qwen3_1p7b_4k"].scaled(batch=2, n_ctx=1000)),
    ("hc_n777", W["llama31_8b_hc_8k"].scaled(batch=3, n_ctx=777)),
    ("ranks_16_48_96_128", W["qwen3_1p7b_4k"].scaled(batch=1, n_q_heads=8, n_kv_heads=4, window=8, n_ctx=333,
                                                  mixed_ranks=True, rank_k_choices=(16, 48, 96, 128),
                                                  rank_v_choices=(16, 48, 96, 128))),
]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("label,w", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("slot0", [0, 3])
def test_compress_q(label, w, slot0, bits):
    announce(f"compress {bits}-bit {label} slot0 {slot0}")
    hc = host_case(w, qbits=bits)
    n = hc.n
    c = max(0, n - 1 - w.window)
    L = gpu_layer(hc, with_codes=False, cap=layout.round_cap(c + slot0))
    for which in "kv":
        src = np.stack([np.stack([(hc.k if which == "k" else hc.v)[b][h][1:1 + c]
                                  for h in range(w.n_kv_heads)]) for b in range(w.batch)])
        B.lrkv_compress(L, 0 if which == "k" else 1, dev(src, "bf16"), c, slot0)
    torch.cuda.synchronize()
    for which in "kv":
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                q, s = read_q(L, which, b, h, c, slot0)
                x = (hc.k if which == "k" else hc.v)[b][h][1:1 + c]
                u = (hc.u_k if which == "k" else hc.u_v)[h]
                check_q_codes(q, s, x, u, bits, f"{label}/{which}/b{b}h{h}/s{slot0}")


# ---------------------------------------------------------------------------
# decode on oracle-made int8 codes
# ---------------------------------------------------------------------------

BASE = W["qwen3_1p7b_4k"].scaled(batch=2, n_q_heads=8, n_kv_heads=2, window=16)

DECODE = [
    ("llama31_8b_n3000_s32", W["llama31_8b_32k"].scaled(batch=1, n_ctx=3000), 32, None),
    ("qwen3_n1000", W["qwen3_1p7b_4k"].scaled(batch=2, n_ctx=1000), 0, None),
    ("hc_n777", W["llama31_8b_hc_8k"].scaled(batch=3, n_ctx=777), 0, None),
    ("mixed_ranks_n2000", W["llama31_8b_32layer"].scaled(batch=2, n_ctx=2000, n_steps=0), 0, None),
    ("ranks_16_48_96_128", BASE.scaled(n_kv_heads=4, n_q_heads=8, n_ctx=500, mixed_ranks=True,
                                       rank_k_choices=(16, 48, 96, 128), rank_v_choices=(16, 48, 96, 128)), 0, None),
    ("n1", BASE.scaled(n_ctx=1), 0, None),
    ("n_window_plus_2", BASE.scaled(n_ctx=18), 0, None),
    ("window0", BASE.scaled(window=0, n_ctx=300), 0, None),
    ("empty_splits", BASE.scaled(n_ctx=17 + 40), 16, None),
    ("many_splits", BASE.scaled(n_ctx=700), 300, None),
    ("gqa_g16", BASE.scaled(n_q_heads=32, n_ctx=400), 0, None),
    ("ragged", BASE.scaled(batch=5, n_ctx=800), 0, [800, 1, 17, 18, 433]),
]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("label,w,S,lens", DECODE, ids=[d[0] for d in DECODE])
def test_decode_q(label, w, S, lens, bits):
    announce(f"decode {bits}-bit {label}: batch {w.batch} n {w.n_ctx} S {S}")
    hc = host_case(w, lens=lens, qbits=bits)
    L = gpu_layer(hc)
    got = gpu_decode(L, hc, n_splits=S, ragged=lens is not None)
    check_decode(got, hc.expected(), "bf16", f"q{bits}_{label}")


@pytest.mark.parametrize("bits", BITS)
def test_decode_q_garbage_past_context(bits):
    """Slots past the context may hold any bytes and any scale bits (NaN here):
    they never reach the result."""
    w = BASE.scaled(n_ctx=17 + 45)
    hc = host_case(w, qbits=bits)
    L = gpu_layer(hc, cap=64)
    want = hc.expected()
    c = hc.n - 1 - w.window
    nan = float("nan")
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            s0 = layout.scale_offset(h, b, L.cap, L.batch)
            L.scales_k[s0 + c:s0 + L.cap] = nan
            L.scales_v[s0 + c:s0 + L.cap] = nan
            for which, ranks, buf in (("k", hc.rk, L.codes_k), ("v", hc.rv, L.codes_v)):
                r = int(ranks[h])
                off = int(layout.code_offsets(ranks, w.batch, L.cap)[h]) + b * L.cap * r
                pos = layout.slot_positions(L.cap, r, which)[c:].ravel()
                if bits == 8:
                    buf[torch.from_numpy(off + pos).cuda()] = -128
                else:  # -8 in the tail's elements only (a byte may also hold a valid slot's)
                    lo, hi = off // 2, (off + L.cap * r) // 2
                    el = layout.unpack_nibbles(buf[lo:hi].cpu().numpy())
                    el[pos] = -8
                    buf[lo:hi] = torch.from_numpy(layout.pack_nibbles(el)).cuda()
    announce(f"decode {bits}-bit with NaN scales and extreme codes past the context")
    check_decode(gpu_decode(L, hc), want, "bf16", f"q{bits}_garbage_tail")


@pytest.mark.parametrize("bits", BITS)
def test_decode_q_peaky(bits):
    w = BASE.scaled(n_ctx=900)
    hc = host_case(w, q_scale=8.0, qbits=bits)
    announce(f"decode {bits}-bit peaky q x8")
    check_decode(gpu_decode(gpu_layer(hc), hc), hc.expected(), "bf16", f"q{bits}_peaky")


# ---------------------------------------------------------------------------
# end to end: prefill compression + anchors + appends, against the oracle's cache
# ---------------------------------------------------------------------------

def rows(w, layer, which):
    a = np.empty((w.batch, w.n_kv_heads, w.n_total, D), np.float32)
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            a[b, h] = synth.unit_kv(w, layer, h, b, which)
    return dev(a, "bf16")


def q_prefill(w, layer, n, bits, extra=0):
    rk, rv = synth.ranks(w, layer)
    bases = layout.pack_bases([synth.basis(w, layer, h, "k", int(rk[h])) for h in range(w.n_kv_heads)],
                              [synth.basis(w, layer, h, "v", int(rv[h])) for h in range(w.n_kv_heads)])
    c = max(0, n - 1 - w.window)
    L = B.Layer.allocate(dtype=DTYPE[bits], batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                         window=w.window, cap=layout.round_cap(c + extra), rank_k=rk, rank_v=rv,
                         bases=dev(bases, "bf16"))
    K, V = rows(w, layer, "k"), rows(w, layer, "v")
    B.lrkv_compress(L, 0, K[:, :, 1:], c, 0)
    B.lrkv_compress(L, 1, V[:, :, 1:], c, 0)
    B.lrkv_store_anchors(L, K[:, :, 0:1], V[:, :, 0:1], 0, 1)
    lo = max(1, n - w.window)
    B.lrkv_store_anchors(L, K[:, :, lo:n], V[:, :, lo:n], lo, n - lo)
    return L, K, V


def oracle_q_units(w, layer, n, units, q, bits):
    rk, rv = synth.ranks(w, layer)
    g = w.group
    out = np.full((w.batch, w.n_q_heads, D), np.nan)
    cpos, apos = oracle.code_positions(n, w.window), oracle.anchor_positions(n, w.window)
    for b, h in units:
        k = synth.unit_kv(w, layer, h, b, "k").astype(np.float64)
        v = synth.unit_kv(w, layer, h, b, "v").astype(np.float64)
        uk = synth.basis(w, layer, h, "k", int(rk[h])).astype(np.float64)
        uv = synth.basis(w, layer, h, "v", int(rv[h])).astype(np.float64)
        ck = code_storage(oracle.oracle_compress(k[cpos], uk), f"q{bits}")
        cv = code_storage(oracle.oracle_compress(v[cpos], uv), f"q{bits}")
        rws = slice(h * g, (h + 1) * g)
        out[b, rws] = oracle.oracle_decode_unit(q[b, rws], uk, uv, ck, cv, k[apos], v[apos],
                                                oracle.default_scale())
    return out


def run_decode(L, w, n, q_np, S):
    q = dev(q_np, "bf16")
    out = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device="cuda")
    B.lrkv_decode_attn(L, n, q, out, oracle.default_scale(), S, B.workspace(L, S))
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def queries(w, layer, step):
    return np.stack([synth.queries(w, layer, step, b) for b in range(w.batch)]).astype(np.float64)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("window", [0, 1, 16])
def test_q_decode_steps_with_append(window, bits):
    w = W["llama31_8b_32layer"].scaled(batch=2, n_ctx=60, n_steps=40, window=window)
    announce(f"{bits}-bit e2e append steps W={window}")
    L, K, V = q_prefill(w, 3, w.n_ctx, bits, extra=w.n_steps)
    units = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    for t in range(1, w.n_steps + 1):
        pos = w.n_ctx + t - 1
        B.lrkv_append(L, K[:, :, pos].contiguous(), V[:, :, pos].contiguous(), pos)
        n = pos + 1
        q = queries(w, 3, t)
        got = run_decode(L, w, n, q, B.lrkv_decode_auto_splits(L, n))
        if t in (1, 2, w.window + 1, w.window + 2, w.n_steps) or t % 9 == 0:
            check_decode(got, oracle_q_units(w, 3, n, units, q, bits), "bf16",
                         f"q{bits}_append_W{window}_t{t}")


@pytest.mark.parametrize("bits", BITS)
def test_q_full_size_llama_32k_sampled(bits):
    """The 32K Llama-3.1-8B-shaped layer with quantised codes, 32 splits: GPU
    prefill compression then one decode, sampled (row, head) units against the
    oracle."""
    w = W["llama31_8b_32k"]
    announce(f"{bits}-bit full size llama31_8b_32k: batch {w.batch} n {w.n_ctx}")
    L, _, _ = q_prefill(w, 0, w.n_ctx, bits)
    q = queries(w, 0, 0)
    got = run_decode(L, w, w.n_ctx, q, 32)
    assert np.all(np.isfinite(got))
    units = [(0, 0), (w.batch // 2, w.n_kv_heads // 2), (w.batch - 1, w.n_kv_heads - 1)]
    check_decode(got, oracle_q_units(w, 0, w.n_ctx, units, q, bits), "bf16", f"q{bits}_full_llama31_8b_32k")
