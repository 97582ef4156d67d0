"""The seeded input generator (no GPU)."""

import numpy as np
import torch

import synth


def test_workload_table_matches_the_five_configs():
    w = synth.WORKLOADS
    assert [x.name for x in w.values()] == ["tiny_f32", "qwen3_1p7b_4k", "llama31_8b_32k",
                                            "llama31_8b_hc_8k", "llama31_8b_32layer"]
    t = w["tiny_f32"]
    assert (t.batch, t.n_q_heads, t.n_kv_heads, t.n_ctx, t.rank_k, t.rank_v, t.window, t.dtype) == \
        (1, 1, 1, 256, 64, 32, 16, "f32")
    q = w["qwen3_1p7b_4k"]
    assert (q.batch, q.n_q_heads, q.n_kv_heads, q.group, q.n_ctx, q.window) == (8, 16, 8, 2, 4096, 64)
    l3 = w["llama31_8b_32k"]
    assert (l3.batch, l3.group, l3.n_ctx, l3.window, l3.n_splits) == (4, 4, 32768, 128, 32)
    hc = w["llama31_8b_hc_8k"]
    assert (hc.batch, hc.n_ctx, hc.rank_k, hc.rank_v, hc.window, hc.tau_k, hc.tau_v) == \
        (64, 8192, 32, 16, 32, 32.0, 16.0)
    l5 = w["llama31_8b_32layer"]
    assert (l5.n_layers, l5.n_steps, l5.n_ctx, l5.n_total, l5.window) == (32, 16, 32768, 32784, 128)


def test_haar_rotation_is_orthogonal_and_seeded():
    w = synth.WORKLOADS["qwen3_1p7b_4k"]
    r1 = synth.rotation(w, 0, 3, "k")
    r2 = synth.rotation(w, 0, 3, "k")
    assert np.array_equal(r1, r2)
    assert np.max(np.abs(r1 @ r1.T - np.eye(128))) < 1e-12
    assert not np.allclose(r1, synth.rotation(w, 0, 3, "v"))


def test_basis_is_orthonormal_top_subspace():
    w = synth.WORKLOADS["tiny_f32"]
    u = synth.basis(w, 0, 0, "k", 64).astype(np.float64)
    assert u.shape == (128, 64)
    assert np.max(np.abs(u.T @ u - np.eye(64))) < 1e-5
    x = synth.calibration_rows(w, 0, 0, "k")
    s = np.linalg.svd(x, compute_uv=False)
    # the captured energy equals the top-64 singular values' energy
    cap = np.sum((x @ u) ** 2)
    assert abs(cap - np.sum(s[:64] ** 2)) / cap < 1e-5


def test_bf16_values_are_representable():
    w = synth.WORKLOADS["qwen3_1p7b_4k"].scaled(n_ctx=64)
    k = synth.unit_kv(w, 0, 1, 2, "k")
    assert k.dtype == np.float32 and k.shape == (64, 128)
    back = torch.from_numpy(k).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(back, k)
    assert np.array_equal(k, synth.unit_kv(w, 0, 1, 2, "k"))
    assert not np.array_equal(k, synth.unit_kv(w, 0, 1, 3, "k"))


def test_spectrum_decay():
    x = synth.unit_kv(synth.WORKLOADS["tiny_f32"], 0, 0, 0, "k").astype(np.float64)
    s = np.linalg.svd(x, compute_uv=False)
    # a decaying spectrum: the top 64 directions hold nearly all the energy
    assert np.sum(s[:64] ** 2) / np.sum(s ** 2) > 0.98


def test_mixed_ranks_from_choices():
    w = synth.WORKLOADS["llama31_8b_32layer"]
    seen_k, seen_v = set(), set()
    for layer in range(32):
        rk, rv = synth.ranks(w, layer)
        assert rk.shape == (8,) and rv.shape == (8,)
        seen_k |= set(rk.tolist())
        seen_v |= set(rv.tolist())
    assert seen_k == {32, 48, 64, 96} and seen_v == {16, 32}
    assert np.array_equal(synth.ranks(w, 5)[0], synth.ranks(w, 5)[0])


def test_32layer_ranks_cover_every_pair_in_mixed_layers():
    """Every (r_k, r_v) pair of the 32-layer workload's choices occurs in a layer
    whose KV heads have other pairs too (so each exact pair runs in a mixed-rank
    decode), (32, 16) included."""
    w = synth.WORKLOADS["llama31_8b_32layer"]
    seen = set()
    for layer in range(w.n_layers):
        rk, rv = synth.ranks(w, layer)
        pairs = set(zip(rk.tolist(), rv.tolist()))
        if len(pairs) > 1:
            seen |= pairs
    assert (32, 16) in seen
    assert seen == {(a, b) for a in w.rank_k_choices for b in w.rank_v_choices}
