"""GPU decode attention against the oracle, element by element, on oracle-made
codes (so the decode kernels are checked independently of the compress kernel).

Sizes are reduced so the oracle finishes in seconds while still spanning many
32-slot blocks with a ragged tail; full-size runs are in test_gpu_e2e.py.
"""

import numpy as np
import pytest

import oracle
import synth
from cases import D, announce, check_decode, dev, gpu_decode, gpu_layer, host_case

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS

# (label, workload at reduced size, n_splits (0 = auto))
REDUCED = [
    ("tiny_f32", W["tiny_f32"], 0),
    ("tiny_f32_s3", W["tiny_f32"], 3),
    ("qwen3_1p7b_n1000", W["qwen3_1p7b_4k"].scaled(batch=2, n_ctx=1000), 0),
    ("llama31_8b_n3000_s32", W["llama31_8b_32k"].scaled(batch=1, n_ctx=3000), 32),
    ("llama31_8b_hc_n777", W["llama31_8b_hc_8k"].scaled(batch=3, n_ctx=777), 0),
    ("llama31_8b_mixed_ranks_n2000", W["llama31_8b_32layer"].scaled(batch=2, n_ctx=2000, n_steps=0), 0),
]


@pytest.mark.parametrize("label,w,S", REDUCED, ids=[r[0] for r in REDUCED])
def test_decode_matches_oracle(label, w, S):
    announce(f"decode {label}: batch {w.batch} Hq {w.n_q_heads} Hkv {w.n_kv_heads} n {w.n_ctx} S {S}")
    hc = host_case(w)
    got = gpu_decode(gpu_layer(hc), hc, n_splits=S)
    check_decode(got, hc.expected(), w.dtype, label)


def test_mixed_ranks_other_layer():
    w = W["llama31_8b_32layer"].scaled(batch=1, n_ctx=1500, n_steps=0)
    hc = host_case(w, layer=7)
    announce(f"decode mixed ranks layer 7 ranks {hc.rk.tolist()} {hc.rv.tolist()}")
    check_decode(gpu_decode(gpu_layer(hc), hc), hc.expected(), "bf16", "mixed_ranks_layer7")


BASE = W["qwen3_1p7b_4k"].scaled(batch=2, n_q_heads=8, n_kv_heads=2, window=16)

EDGE = [
    ("n1", BASE.scaled(n_ctx=1), 0),
    ("n_window_plus_1", BASE.scaled(n_ctx=17), 0),
    ("n_window_plus_2", BASE.scaled(n_ctx=18), 0),
    ("one_block_exact", BASE.scaled(n_ctx=17 + 32), 0),
    ("window0", BASE.scaled(window=0, n_ctx=300), 0),
    ("window0_n1", BASE.scaled(window=0, n_ctx=1), 0),
    ("empty_splits", BASE.scaled(n_ctx=17 + 40), 16),
    ("single_split", BASE.scaled(n_ctx=700), 1),
    ("many_splits", BASE.scaled(n_ctx=700), 300),
    ("mha_g1", BASE.scaled(n_q_heads=2, n_ctx=400), 0),
    ("gqa_g8", BASE.scaled(n_q_heads=16, n_ctx=400), 0),
    ("gqa_g16", BASE.scaled(n_q_heads=32, n_ctx=400), 0),
    ("wide_window", BASE.scaled(window=300, n_ctx=1000), 0),
    # value rank 48: rv / 4 = 12 threads a split row does not divide the combine's
    # 128 threads, so a round holds P whole rows of 10 splits; every split here
    # has code blocks (one round of the single-version merge, and more rounds
    # than one of the general merge)
    ("rv48_s42", BASE.scaled(rank_v=48, n_ctx=3000), 42),
    ("rv48_s165", BASE.scaled(rank_v=48, n_ctx=6000), 165),
    ("ranks_16_48_96_128", BASE.scaled(n_kv_heads=4, n_q_heads=8, n_ctx=500, mixed_ranks=True,
                                       rank_k_choices=(16, 48, 96, 128), rank_v_choices=(16, 48, 96, 128)), 0),
    ("rank128_f32", BASE.scaled(dtype="f32", rank_k=128, rank_v=128, n_ctx=300), 0),
    ("ranks_f32_mixed", BASE.scaled(dtype="f32", n_kv_heads=4, n_q_heads=8, n_ctx=333, mixed_ranks=True,
                                    rank_k_choices=(16, 48, 96), rank_v_choices=(16, 48, 96)), 0),
]


@pytest.mark.parametrize("label,w,S", EDGE, ids=[e[0] for e in EDGE])
def test_decode_edge_cases(label, w, S):
    announce(f"decode edge {label}: n {w.n_ctx} W {w.window} g {w.group} S {S}")
    hc = host_case(w)
    check_decode(gpu_decode(gpu_layer(hc), hc, n_splits=S), hc.expected(), w.dtype, label)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_peaky_attention(dtype):
    w = BASE.scaled(dtype=dtype, n_ctx=900)
    announce(f"decode peaky q x8 {dtype}")
    hc = host_case(w, q_scale=8.0)
    check_decode(gpu_decode(gpu_layer(hc), hc), hc.expected(), dtype, f"peaky_{dtype}")


def test_ragged_batch():
    w = BASE.scaled(batch=5, n_ctx=800)
    lens = [800, 1, 17, 18, 433]
    announce(f"decode ragged lens {lens}")
    hc = host_case(w, lens=lens)
    check_decode(gpu_decode(gpu_layer(hc), hc, ragged=True), hc.expected(), "bf16", "ragged")


def test_custom_scale():
    w = BASE.scaled(n_ctx=300)
    hc = host_case(w)
    announce("decode custom sm_scale 0.05")
    check_decode(gpu_decode(gpu_layer(hc), hc, scale=0.05), hc.expected(scale=0.05), "bf16", "scale0.05")


def test_bitwise_reproducible_and_split_invariant():
    w = W["qwen3_1p7b_4k"].scaled(batch=2, n_ctx=2500)
    announce("decode determinism")
    hc = host_case(w)
    L = gpu_layer(hc)
    a = gpu_decode(L, hc, n_splits=7)
    b = gpu_decode(L, hc, n_splits=7)
    assert np.array_equal(a, b), "same n_splits must give identical bits"
    want = hc.expected()
    for S in (1, 5, 64):
        check_decode(gpu_decode(L, hc, n_splits=S), want, "bf16", f"splits{S}")


@pytest.mark.parametrize("S,window,ragged", [(3, 64, False), (40, 64, True), (300, 600, False)])
def test_two_stage_entry_points(S, window, ragged):
    """Stage 1 and stage 2 called on their own (lrkv_decode_partials, then
    lrkv_decode_combine with the same context lengths) give the whole call's
    bits.  S = 40 and S = 300 take the merge past the terms it loads up front;
    window 600 puts anchor sums on many splits; the ragged case gives rows
    different anchor splits."""
    import torch
    from rank_kv_cache_lrkv_amd import binding as B
    w = W["qwen3_1p7b_4k"].scaled(batch=3 if ragged else 2, n_ctx=2500, window=window)
    announce(f"two-stage entry points S={S} W={window} ragged={ragged}")
    hc = host_case(w, lens=[2500, 700, 40] if ragged else None)
    L = gpu_layer(hc)
    whole = gpu_decode(L, hc, n_splits=S, ragged=ragged)
    q = dev(hc.q, w.dtype)
    lens = torch.tensor(hc.lens, dtype=torch.int32, device="cuda") if ragged else None
    ws = B.workspace(L, S)
    two = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device="cuda")
    B.lrkv_decode_partials(L, hc.n, q, oracle.default_scale(), S, ws, ctx_lens=lens)
    B.lrkv_decode_combine(L, hc.n, S, ws, two, ctx_lens=lens)
    torch.cuda.synchronize()
    assert np.array_equal(two.cpu().numpy().astype(np.float64), whole), "stage 1 + stage 2 != whole call"
    check_decode(whole, hc.expected(), "bf16", f"two-stage S{S}")
