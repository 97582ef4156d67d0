"""GPU prefill compression and cache maintenance against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import D, announce, dev, gpu_layer, host_case
from rank_kv_cache_lrkv_amd import binding as B, layout

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (normal range)."""
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def upload_rows(hc, which, n):
    """[batch][Hkv][n][128] device tensor of the first n rows."""
    src = hc.k if which == "k" else hc.v
    a = np.stack([np.stack([src[b][h][:n] for h in range(hc.w.n_kv_heads)]) for b in range(hc.w.batch)])
    return dev(a, hc.w.dtype)


def read_codes(L, hc, which, b, h, n):
    from cases import torch_dtype  # noqa: F401
    r = int((hc.rk if which == "k" else hc.rv)[h])
    off = layout.code_offsets(hc.rk if which == "k" else hc.rv, hc.w.batch, L.cap)[h] + b * L.cap * r
    flat = (L.codes_k if which == "k" else L.codes_v)[off:off + L.cap * r].float().cpu().numpy()
    return layout.unpack_codes(flat.astype(np.float64), n, r, which)


def check_codes(got, x, u, dtype, label):
    """float32 storage: max abs error <= 1e-5.  bf16 storage: every code within
    the float32 dot-product error bound plus half a bf16 spacing of the exact
    value (|x.u - fl32(x.u)| <= gamma_128 * sum|x_i u_i|, gamma_n = n u/(1 - n u),
    u = 2^-24, then round to nearest), and >= 99% of codes bit-equal to the exact
    value rounded to bf16 (a sanity check: at rank 128 the trailing directions
    hold small codes whose roundings a float32 accumulation flips ~0.2% of the
    time, the rate a sequential float32 FMA emulation also shows)."""
    exact = oracle.oracle_compress(x, u)
    if dtype == "f32":
        e = float(np.max(np.abs(got - exact))) if got.size else 0.0
        print(f"[parity] {label}: compress max abs err {e:.3e}", flush=True)
        assert e <= 1e-5, (label, e)
        return
    if not got.size:
        return
    rne = oracle.bf16_round(exact)
    uu = 2.0 ** -24
    gamma = D * uu / (1 - D * uu)
    acc_bound = gamma * (np.abs(x) @ np.abs(u))
    bound = acc_bound + 0.5 * bf16_ulp(np.abs(exact) + acc_bound)
    worst = float(np.max(np.abs(got - exact) / bound))
    equal = float(np.mean(got == rne))
    print(f"[parity] {label}: compress worst {worst:.3f} of bound, bit-equal to RNE {equal:.5f}", flush=True)
    assert worst <= 1.0, (label, worst)
    assert equal >= 0.99, (label, equal)


CASES = [
    ("tiny_f32", W["tiny_f32"]),
    ("qwen3_n1000", W["qwen3_1p7b_4k"].scaled(batch=2, n_ctx=1000)),
    ("hc_n777", W["llama31_8b_hc_8k"].scaled(batch=3, n_ctx=777)),
    ("mixed_ranks_n700", W["llama31_8b_32layer"].scaled(batch=2, n_ctx=700, n_steps=0)),
    ("ranks_16_48_96_128", W["qwen3_1p7b_4k"].scaled(batch=1, n_q_heads=8, n_kv_heads=4, window=8, n_ctx=333,
                                                  mixed_ranks=True, rank_k_choices=(16, 48, 96, 128),
                                                  rank_v_choices=(16, 48, 96, 128))),
]


@pytest.mark.parametrize("label,w", CASES, ids=[c[0] for c in CASES])
def test_compress_matches_oracle(label, w):
    announce(f"compress {label}")
    hc = host_case(w)
    n, Wn = hc.n, w.window
    c = max(0, n - 1 - Wn)
    L = gpu_layer(hc, with_codes=False)
    for which in "kv":
        x = upload_rows(hc, which, n)
        B.lrkv_compress(L, 0 if which == "k" else 1, x[:, :, 1:1 + c], c, 0)
    torch.cuda.synchronize()
    for which in "kv":
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                got = read_codes(L, hc, which, b, h, c)
                src = (hc.k if which == "k" else hc.v)[b][h][1:1 + c]
                u = (hc.u_k if which == "k" else hc.u_v)[h]
                check_codes(got, src, u, w.dtype, f"{label}/{which}/b{b}h{h}")


def test_compress_slot_range_only():
    """Writes land in [slot0, slot0 + n_tok) and nowhere else (canary fill)."""
    w = W["qwen3_1p7b_4k"].scaled(batch=2, n_q_heads=4, n_kv_heads=2, n_ctx=200, window=8)
    hc = host_case(w)
    L = gpu_layer(hc, with_codes=False, cap=256)
    L.codes_k.fill_(7.0)
    L.codes_v.fill_(7.0)
    x = upload_rows(hc, "k", 200)
    announce("compress slot range 37..37+45 with canaries")
    B.lrkv_compress(L, 0, x[:, :, 10:55], 45, 37)
    B.lrkv_compress(L, 1, upload_rows(hc, "v", 200)[:, :, 10:55], 45, 37)
    torch.cuda.synchronize()
    for which in "kv":
        for b in range(2):
            for h in range(2):
                allc = read_codes(L, hc, which, b, h, 256)
                assert np.all(allc[:37] == 7.0) and np.all(allc[82:] == 7.0)
                src = (hc.k if which == "k" else hc.v)[b][h][10:55]
                check_codes(allc[37:82], src, (hc.u_k if which == "k" else hc.u_v)[h], "bf16",
                            f"range/{which}/b{b}h{h}")


def test_store_anchors_ring():
    w = W["qwen3_1p7b_4k"].scaled(batch=2, n_q_heads=4, n_kv_heads=2, n_ctx=50, window=8)
    hc = host_case(w)
    L = gpu_layer(hc, with_codes=False)
    k, v = upload_rows(hc, "k", 50), upload_rows(hc, "v", 50)
    announce("store anchors: token 0 and the last 8 of 50")
    B.lrkv_store_anchors(L, k[:, :, 0:1], v[:, :, 0:1], 0, 1)
    B.lrkv_store_anchors(L, k[:, :, 42:50], v[:, :, 42:50], 42, 8)
    torch.cuda.synchronize()
    ak = L.anchor_k.float().cpu().numpy()
    av = L.anchor_v.float().cpu().numpy()
    for b in range(2):
        for h in range(2):
            for p in [0, *range(42, 50)]:
                s = layout.anchor_slot(p, 8)
                assert np.array_equal(ak[b, h, s], hc.k[b][h][p])
                assert np.array_equal(av[b, h, s], hc.v[b][h][p])


APPEND = [
    ("bf16_W4_mixed", W["qwen3_1p7b_4k"].scaled(batch=2, n_q_heads=8, n_kv_heads=4, window=4, n_ctx=0,
                                                 n_steps=70, mixed_ranks=True, rank_k_choices=(16, 48, 96, 128),
                                                 rank_v_choices=(16, 32, 128))),
    ("bf16_W0", W["llama31_8b_32layer"].scaled(batch=2, window=0, n_ctx=0, n_steps=40)),
    ("f32_W4", W["tiny_f32"].scaled(window=4, n_ctx=0, n_steps=45)),
]


@pytest.mark.parametrize("label,w", APPEND, ids=[a[0] for a in APPEND])
def test_append_codes_match_oracle(label, w):
    """Cache maintenance token by token from position 0: every code slot an append
    fills holds the projection of the token that left the window (of the new
    token when W = 0), within the compress bar, and the anchor ring holds the
    last W tokens exactly."""
    announce(f"append codes {label}")
    hc = host_case(w, n=w.n_steps)
    n, Wn = w.n_steps, w.window
    L = gpu_layer(hc, with_codes=False, cap=layout.round_cap(n))
    k, v = upload_rows(hc, "k", n), upload_rows(hc, "v", n)
    for pos in range(n):
        B.lrkv_append(L, k[:, :, pos].contiguous(), v[:, :, pos].contiguous(), pos)
    torch.cuda.synchronize()
    c = max(0, n - 1 - Wn)  # code slots filled: tokens 1 .. n - W - 1
    for which in "kv":
        for b in range(w.batch):
            for h in range(w.n_kv_heads):
                got = read_codes(L, hc, which, b, h, c)
                src = (hc.k if which == "k" else hc.v)[b][h][1:1 + c]
                check_codes(got, src, (hc.u_k if which == "k" else hc.u_v)[h], w.dtype, f"{label}/{which}/b{b}h{h}")
    ak = L.anchor_k.float().cpu().numpy()
    av = L.anchor_v.float().cpu().numpy()
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            for p in oracle.anchor_positions(n, Wn):
                s = layout.anchor_slot(int(p), Wn)
                assert np.array_equal(ak[b, h, s], hc.k[b][h][p]) and np.array_equal(av[b, h, s], hc.v[b][h][p])
