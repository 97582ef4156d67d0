"""Pins of the CPU oracle against things other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
what the pages or the mathematics fix.  test_oracle.py runs them all;
test_oracle_mutants.py plants plausible mistakes in the oracle and checks that
at least one pin catches each.

References used here (none shares code with the oracle):
* torch.nn.functional.scaled_dot_product_attention in float64 on the CPU;
* brute force: the cache reconstructed token by token, then softmax attention
  written as explicit Python loops with math.exp;
* torch's float32 -> bfloat16 conversion for the rounding helper;
* closed forms and invariances of softmax attention.
"""

from __future__ import annotations

import json
import math
import os

import numpy as np
import torch

import oracle

D = 128
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------

def sdpa(q, keys, values, scale):
    """Library softmax attention, float64 CPU: q (g, d), keys/values (n, d) shared by all g rows."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None, :, None, :]
    g = qt.shape[1]
    kt = torch.from_numpy(np.asarray(keys, np.float64))[None, None].expand(1, g, -1, -1)
    vt = torch.from_numpy(np.asarray(values, np.float64))[None, None].expand(1, g, -1, -1)
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=scale)
    return out[0, :, 0, :].numpy()


def brute_attention(q_row, keys, values, scale):
    """Softmax attention for one query row with explicit loops."""
    n = len(keys)
    scores = [scale * sum(float(q_row[i]) * float(keys[j][i]) for i in range(len(q_row))) for j in range(n)]
    top = max(scores)
    w = [math.exp(s - top) for s in scores]
    tot = sum(w)
    d = len(values[0])
    out = [sum(w[j] * float(values[j][i]) for j in range(n)) / tot for i in range(d)]
    return np.array(out), np.array(w) / tot


def reconstruct(codes, u):
    """Full-dim rows back from codes, one token at a time: x_hat_j = U c_j."""
    return np.stack([np.asarray(u, np.float64) @ np.asarray(c, np.float64) for c in codes]) \
        if len(codes) else np.zeros((0, D))


# ---------------------------------------------------------------------------
# random inputs for the pins
# ---------------------------------------------------------------------------

def orthonormal(rng, r):
    a = rng.standard_normal((D, D))
    qm, _ = np.linalg.qr(a)
    return qm[:, :r]


def random_unit(rng, n, window, r_k, r_v, g=2, q_scale=1.0, u_k=None, u_v=None):
    """A random cache for one KV head at n tokens, split into codes and anchors
    by the oracle's own partition.  Returns dict of arrays (float64)."""
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, D))
    q = rng.standard_normal((g, D)) * q_scale
    u_k = orthonormal(rng, r_k) if u_k is None else u_k
    u_v = orthonormal(rng, r_v) if u_v is None else u_v
    cpos = oracle.code_positions(n, window)
    apos = oracle.anchor_positions(n, window)
    return dict(q=q, k=k, v=v, u_k=u_k, u_v=u_v, cpos=cpos, apos=apos,
                c_k=k[cpos] @ u_k, c_v=v[cpos] @ u_v, k_a=k[apos], v_a=v[apos])


def run_unit(u, scale=None, return_p=False):
    scale = oracle.default_scale() if scale is None else scale
    return oracle.oracle_decode_unit(u["q"], u["u_k"], u["u_v"], u["c_k"], u["c_v"],
                                     u["k_a"], u["v_a"], scale, return_p=return_p)


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


# ---------------------------------------------------------------------------
# pins
# ---------------------------------------------------------------------------

def pin_bf16_round_matches_torch():
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0], np.float32),
    ])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, ref), "bf16 rounding disagrees with torch's conversion"


def pin_bf16_round_ties():
    # spacing of bf16 in [1, 2) is 2**-7; halfway cases go to the even neighbour
    cases = {1 + 2**-8: 1.0, 1 + 3 * 2**-8: 1 + 2**-6, -(1 + 2**-8): -1.0,
             1 + 2**-8 + 2**-20: 1 + 2**-7, 2**-133 * 1.5: 2**-132, 3.0: 3.0}
    for x, want in cases.items():
        got = float(oracle.bf16_round(np.array([x]))[0])
        assert got == want, (x, got, want)


def pin_partition():
    for n in [1, 2, 3, 16, 17, 18, 19, 100, 257]:
        for w in [0, 1, 16, 64]:
            a = oracle.anchor_positions(n, w)
            c = oracle.code_positions(n, w)
            allp = np.sort(np.concatenate([a, c]))
            assert np.array_equal(allp, np.arange(n)), (n, w)
            assert len(a) == min(n, 1 + w), (n, w, len(a))
            assert a[0] == 0
            if n > 1 and w > 0:
                assert a[-1] == n - 1, "the decode token itself must be a full-rank anchor"
            assert len(c) == max(0, n - 1 - w)


def pin_plumbing_identity_basis():
    """Blog section 04 plumbing check: an uncompressed cache routed through the
    path (r = d, U = I) reproduces full attention."""
    rng = np.random.default_rng(1)
    eye = np.eye(D)
    u = random_unit(rng, 200, 16, D, D, g=3, u_k=eye, u_v=eye)
    got = run_unit(u)
    want = sdpa(u["q"], u["k"], u["v"], oracle.default_scale())
    assert rel(got, want) < 1e-12, rel(got, want)


def pin_plumbing_orthogonal_basis():
    """Same check with a full-rank non-symmetric orthogonal basis (r = d)."""
    rng = np.random.default_rng(2)
    u_k = orthonormal(rng, D)
    u_v = orthonormal(rng, D)
    u = random_unit(rng, 150, 8, D, D, g=2, u_k=u_k, u_v=u_v)
    got = run_unit(u)
    want = sdpa(u["q"], u["k"], u["v"], oracle.default_scale())
    assert rel(got, want) < 1e-12, rel(got, want)


def pin_brute_force_tiny():
    """Low rank: the oracle equals attention over the reconstructed cache,
    computed with explicit loops, including the weights."""
    rng = np.random.default_rng(3)
    for (n, w, rk, rv, g) in [(12, 3, 16, 32, 2), (7, 0, 48, 16, 1), (9, 20, 32, 16, 3), (30, 5, 96, 64, 2)]:
        u = random_unit(rng, n, w, rk, rv, g=g, q_scale=3.0)
        out, p = run_unit(u, return_p=True)
        keys = np.concatenate([reconstruct(u["c_k"], u["u_k"]), u["k_a"]])
        vals = np.concatenate([reconstruct(u["c_v"], u["u_v"]), u["v_a"]])
        for i in range(g):
            bo, bp = brute_attention(u["q"][i], keys, vals, oracle.default_scale())
            assert rel(out[i], bo) < 1e-12, (n, w, rk, rv, rel(out[i], bo))
            assert np.max(np.abs(p[i] - bp)) < 1e-14


def pin_sdpa_low_rank():
    """Low rank at larger n against the library routine over the reconstructed cache."""
    rng = np.random.default_rng(4)
    for (n, w, rk, rv, g, qs) in [(300, 16, 64, 32, 4, 1.0), (513, 64, 32, 16, 2, 8.0),
                                 (64, 100, 64, 32, 1, 1.0), (1000, 0, 128, 16, 8, 4.0)]:
        u = random_unit(rng, n, w, rk, rv, g=g, q_scale=qs)
        got = run_unit(u)
        keys = np.concatenate([u["c_k"] @ u["u_k"].T, u["k_a"]])
        vals = np.concatenate([u["c_v"] @ u["u_v"].T, u["v_a"]])
        want = sdpa(u["q"], keys, vals, oracle.default_scale())
        assert rel(got, want) < 1e-12, (n, w, rk, rv, rel(got, want))


def pin_code_space_identity():
    """(U^T q).(U^T k) = q.(U U^T k) for any basis: ties scoring and orientation."""
    rng = np.random.default_rng(5)
    for r in [16, 48, 128]:
        u = orthonormal(rng, r)
        q = rng.standard_normal((3, D))
        k = rng.standard_normal((10, D))
        s_code = oracle.code_scores(oracle.project_query(q, u), oracle.oracle_compress(k, u), 1.0)
        s_full = q @ (u @ u.T @ k.T)
        assert np.max(np.abs(s_code - s_full)) < 1e-11


def pin_weights_sum_to_one():
    rng = np.random.default_rng(6)
    for qs in [1.0, 30.0]:
        u = random_unit(rng, 400, 32, 64, 32, g=4, q_scale=qs)
        _, p = run_unit(u, return_p=True)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1)) < 1e-14


def pin_constant_values():
    """Every value (reconstructed or anchor) equal to v0 -> out = v0."""
    rng = np.random.default_rng(7)
    u = random_unit(rng, 120, 10, 64, 32, g=2, q_scale=5.0)
    z = rng.standard_normal(32)
    v0 = u["u_v"] @ z
    u["c_v"] = np.tile(z, (len(u["cpos"]), 1))
    u["v_a"] = np.tile(v0, (len(u["apos"]), 1))
    got = run_unit(u)
    assert np.max(np.abs(got - v0[None, :])) < 1e-13


def pin_anchors_only():
    """n <= 1 + W: nothing is compressed; full attention over the n tokens."""
    rng = np.random.default_rng(8)
    u = random_unit(rng, 40, 64, 32, 16, g=2)
    assert len(u["cpos"]) == 0
    got = run_unit(u)
    want = sdpa(u["q"], u["k"], u["v"], oracle.default_scale())
    assert rel(got, want) < 1e-12


def pin_single_token():
    rng = np.random.default_rng(9)
    u = random_unit(rng, 1, 16, 64, 32, g=3)
    got = run_unit(u)
    assert np.max(np.abs(got - u["v"][0][None, :])) < 1e-15


def pin_zero_query():
    """q = 0: all scores equal, out is the mean of all (reconstructed) values."""
    rng = np.random.default_rng(10)
    u = random_unit(rng, 90, 7, 48, 32, g=2)
    u["q"] = np.zeros_like(u["q"])
    got = run_unit(u)
    mean = (u["c_v"].sum(axis=0) @ u["u_v"].T + u["v_a"].sum(axis=0)) / 90
    assert np.max(np.abs(got - mean[None, :])) < 1e-14


def pin_basis_sign_and_token_order():
    rng = np.random.default_rng(12)
    u = random_unit(rng, 200, 12, 64, 32, g=2)
    base = run_unit(u)
    flipped = dict(u)
    sk = np.where(rng.random(64) < 0.5, -1.0, 1.0)
    sv = np.where(rng.random(32) < 0.5, -1.0, 1.0)
    flipped["u_k"] = u["u_k"] * sk
    flipped["c_k"] = u["c_k"] * sk
    flipped["u_v"] = u["u_v"] * sv
    flipped["c_v"] = u["c_v"] * sv
    assert rel(run_unit(flipped), base) < 1e-13
    perm = dict(u)
    pc = rng.permutation(len(u["cpos"]))
    pa = rng.permutation(len(u["apos"]))
    perm["c_k"], perm["c_v"] = u["c_k"][pc], u["c_v"][pc]
    perm["k_a"], perm["v_a"] = u["k_a"][pa], u["v_a"][pa]
    assert rel(run_unit(perm), base) < 1e-13


def pin_scale_is_head_dim():
    """The score scale is 1/sqrt(128) whatever the rank: at r = d with U = I the
    oracle must agree with the library's default-scaled attention."""
    assert oracle.default_scale() == 1.0 / math.sqrt(128)
    rng = np.random.default_rng(13)
    eye = np.eye(D)
    u = random_unit(rng, 64, 4, D, D, g=1, q_scale=4.0, u_k=eye, u_v=eye)
    qt = torch.from_numpy(u["q"])[None, :, None, :]
    kt = torch.from_numpy(u["k"])[None, None]
    vt = torch.from_numpy(u["v"])[None, None]
    want = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[0, :, 0].numpy()
    assert rel(run_unit(u), want) < 1e-12


def pin_compress_closed_forms():
    rng = np.random.default_rng(14)
    x = rng.standard_normal((50, D))
    assert np.array_equal(oracle.oracle_compress(x, np.eye(D)), x)
    for r in [16, 64]:
        u = orthonormal(rng, r)
        z = rng.standard_normal((40, r))
        assert np.max(np.abs(oracle.oracle_compress(z @ u.T, u) - z)) < 1e-13
    # calibration: the columns of X U have norms equal to the top singular values
    xc = rng.standard_normal((256, D)) * np.exp(-np.arange(D) / 16.0)
    _, s, vt = np.linalg.svd(xc, full_matrices=False)
    c = oracle.oracle_compress(xc, vt[:32].T)
    assert np.max(np.abs(np.linalg.norm(c, axis=0) - s[:32]) / s[:32]) < 1e-12
    # rows of different shapes of the same data give the same codes
    assert np.array_equal(oracle.oracle_compress(x[:7], np.eye(D)[:, :16]), x[:7, :16])


def pin_kv_bytes_ojakv():
    g = json.load(open(os.path.join(GOLDEN, "ojakv_kv_bytes.json")))
    nbytes = oracle.full_kv_bytes(g["n_layers"], g["n_kv_heads"], g["n_tokens"], g["batch"],
                                  g["head_dim"], g["elem_bytes"])
    assert nbytes == 16 * 2**30
    assert abs(nbytes / 1e9 - g["stated_gb"]) / g["stated_gb"] < 0.1


def pin_payload_ratios_blog():
    g = json.load(open(os.path.join(GOLDEN, "blog_payload_ratios.json")))
    full = 2 * D * 2
    for case in g["cases"]:
        if "ratio" in case:
            n = 100000
            per_tok = oracle.compressed_unit_bytes(n, 0, case["r_k"], case["r_v"]) / n
            ratio = full / per_tok
            assert abs(ratio - case["ratio"]) <= case["tolerance"] * case["ratio"] + 0.04, (case, ratio)
        else:
            assert case["r_v"] / D == case["value_fraction"]
    # anchors are read at full width: at n <= 1 + W nothing is saved
    assert oracle.compressed_unit_bytes(50, 64, 32, 16) == 50 * full




def pin_q8_hand_examples():
    """Int8 rows whose scale comes out a power of two, so every quotient is exact
    and the rounding rule shows: halves go to the even integer."""
    x = np.array([[127.0, -63.5, 0.25, 0.0, 62.5], [254.0, 1.0, -3.0, 5.0, -254.0]], np.float32)
    q, s = oracle.quantize_codes_q8(x)
    assert s.tolist() == [1.0, 2.0], s
    assert q[0].tolist() == [127, -64, 0, 0, 62], q[0]
    assert q[1].tolist() == [127, 0, -2, 2, -127], q[1]


def pin_q8_invariants():
    """Every non-zero row reaches +-127 at its largest entry, each entry is
    reconstructed to within half a step, signs are kept, a zero row stays zero,
    and a power-of-two factor moves into the scale only."""
    rng = np.random.default_rng(21)
    x = (rng.standard_normal((200, 48)) * rng.uniform(0.01, 50, (200, 1))).astype(np.float32)
    x[7] = 0
    q, s = oracle.quantize_codes_q8(x)
    assert s[7] == 0 and not q[7].any()
    nz = s > 0
    assert np.all(np.abs(q[nz].astype(int)).max(axis=1) == 127)
    err = np.abs(oracle.dequantize_codes_q8(q, s) - x.astype(np.float64))
    assert np.all(err <= (0.5 + 1e-5) * s.astype(np.float64)[:, None])
    assert np.all((np.sign(q) == np.sign(x)) | (q == 0))
    q2, s2 = oracle.quantize_codes_q8(x * np.float32(8))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(8))


def pin_q8_unit_bytes():
    """An int8 code row is r bytes plus a 4-byte scale: r 64/32 reads 104 bytes
    per compressed token per KV head instead of 192."""
    n, w = 1000, 16
    c, a = len(oracle.code_positions(n, w)), len(oracle.anchor_positions(n, w))
    assert oracle.compressed_unit_bytes(n, w, 64, 32, q8=True) == c * 104 + a * 512
    assert oracle.compressed_unit_bytes(n, w, 64, 32) == c * 192 + a * 512


def pin_q4_hand_examples():
    """4-bit rows whose scale is a power of two: halves go to the even integer,
    the extremes land on +-7."""
    x = np.array([[7.0, -3.5, 0.25, 0.0, 2.5], [14.0, 1.0, -3.0, 5.0, -14.0]], np.float32)
    q, s = oracle.quantize_codes_q4(x)
    assert s.tolist() == [1.0, 2.0], s
    assert q[0].tolist() == [7, -4, 0, 0, 2], q[0]
    assert q[1].tolist() == [7, 0, -2, 2, -7], q[1]


def pin_q4_invariants():
    """As for int8 with 7 steps: the largest entry of a non-zero row is +-7,
    every entry within half a step, signs kept, zero rows zero, powers of two
    move into the scale only; and a 4-bit code is never finer than the int8 one."""
    rng = np.random.default_rng(22)
    x = (rng.standard_normal((200, 48)) * rng.uniform(0.01, 50, (200, 1))).astype(np.float32)
    x[3] = 0
    q, s = oracle.quantize_codes_q4(x)
    assert s[3] == 0 and not q[3].any()
    nz = s > 0
    assert np.all(np.abs(q[nz].astype(int)).max(axis=1) == 7)
    assert np.all(np.abs(q.astype(int)) <= 7)
    err = np.abs(oracle.dequantize_codes_q4(q, s) - x.astype(np.float64))
    assert np.all(err <= (0.5 + 1e-5) * s.astype(np.float64)[:, None])
    assert np.all((np.sign(q) == np.sign(x)) | (q == 0))
    q2, s2 = oracle.quantize_codes_q4(x * np.float32(4))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(4))
    q8, s8 = oracle.quantize_codes_q8(x)
    e8 = np.abs(oracle.dequantize_codes_q8(q8, s8) - x.astype(np.float64)).max()
    assert e8 < err.max()


def pin_q4_unit_bytes():
    """A 4-bit code row is r / 2 bytes plus a 4-byte scale: 56 bytes per
    compressed token per KV head at r 64/32."""
    n, w = 1000, 16
    c, a = len(oracle.code_positions(n, w)), len(oracle.anchor_positions(n, w))
    assert oracle.compressed_unit_bytes(n, w, 64, 32, q4=True) == c * 56 + a * 512


def pin_layer_gqa_sdpa():
    """Whole-layer decode with distinct KV heads against the library's GQA
    attention (query head i reads KV head i // g)."""
    rng = np.random.default_rng(15)
    batch, n_kv, g, n, w = 2, 3, 2, 70, 5
    cpos, apos = oracle.code_positions(n, w), oracle.anchor_positions(n, w)
    q = rng.standard_normal((batch, n_kv * g, D)) * 2
    bk = [orthonormal(rng, rk) for rk in (16, 32, 64)]
    bv = [orthonormal(rng, rv) for rv in (32, 16, 48)]
    K = rng.standard_normal((batch, n_kv, n, D))
    V = rng.standard_normal((batch, n_kv, n, D))
    ck = [[K[b, h][cpos] @ bk[h] for h in range(n_kv)] for b in range(batch)]
    cv = [[V[b, h][cpos] @ bv[h] for h in range(n_kv)] for b in range(batch)]
    ka = [[K[b, h][apos] for h in range(n_kv)] for b in range(batch)]
    va = [[V[b, h][apos] for h in range(n_kv)] for b in range(batch)]
    got = oracle.oracle_decode_layer(q, bk, bv, ck, cv, ka, va)
    Kh = np.empty((batch, n_kv, n, D))
    Vh = np.empty((batch, n_kv, n, D))
    for b in range(batch):
        for h in range(n_kv):
            Kh[b, h][cpos] = ck[b][h] @ bk[h].T
            Kh[b, h][apos] = ka[b][h]
            Vh[b, h][cpos] = cv[b][h] @ bv[h].T
            Vh[b, h][apos] = va[b][h]
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, :, None, :], torch.from_numpy(Kh), torch.from_numpy(Vh),
        enable_gqa=True)[:, :, 0, :].numpy()
    assert rel(got, want) < 1e-12, rel(got, want)


# ---------------------------------------------------------------------------
# online basis adaptation (Oja's subspace rule) and versioned codes
# ---------------------------------------------------------------------------

def _spectrum_rows(rng, n, sig, rot):
    """n rows whose second-moment matrix is about rot diag(sig^2) rot^T."""
    return (rng.standard_normal((n, len(sig))) * sig[None, :]) @ rot.T


def pin_oja_fixed_point():
    """If u spans an invariant subspace of the batch's second-moment matrix C,
    the rule's step is zero (C u = u u^T C u), for any rotation of that
    subspace: the update returns u itself."""
    rng = np.random.default_rng(31)
    rot = orthonormal(rng, D)
    sig = np.exp(-np.arange(D) / 16.0)
    x = np.sqrt(D) * (sig[:, None] * rot.T)        # x^T x / D = rot diag(sig^2) rot^T exactly
    for r in (1, 16, 64):
        spin = orthonormal(rng, r)[:r, :r] if r > 1 else np.ones((1, 1))
        u = rot[:, :r] @ spin
        u = oracle.orthonormalise(u)               # exact orthonormal columns, same span
        got = oracle.oja_update(u, x, 0.7)
        # the step vanishes; the QR sign convention may flip no column of an
        # already-orthonormal u whose R is the identity
        assert np.max(np.abs(got - u)) < 1e-10, (r, np.max(np.abs(got - u)))


def pin_oja_converges_to_top_subspace():
    """Repeated steps on one batch with a spectral gap converge to the span of
    the top-r eigenvectors of x^T x (LAPACK's symmetric eigensolver)."""
    rng = np.random.default_rng(32)
    rot = orthonormal(rng, D)
    sig = np.concatenate([np.linspace(2.0, 1.0, 8), 0.3 * np.exp(-np.arange(D - 8) / 16.0)])
    x = _spectrum_rows(rng, 3000, sig, rot)
    w, vecs = np.linalg.eigh(x.T @ x / len(x))
    top = vecs[:, np.argsort(w)[::-1][:8]]
    u = orthonormal(rng, 8)
    # step 0.2: every mode outside the subspace shrinks by 1 - 0.2 (l_in - l_out), in (0, 1)
    for _ in range(200):
        u = oracle.oja_update(u, x, 0.2)
    dist = np.linalg.norm(u @ u.T - top @ top.T)
    assert dist < 1e-8, dist
    assert np.max(np.abs(u.T @ u - np.eye(8))) < 1e-12


def pin_oja_single_unit_textbook():
    """r = 1 and one row: Oja's single-neuron rule w + eta y (x - y w), y = x.w,
    then normalised."""
    rng = np.random.default_rng(33)
    w = rng.standard_normal(D)
    w /= np.linalg.norm(w)
    x = rng.standard_normal(D)
    y = float(x @ w)
    want = w + 0.05 * y * (x - y * w)
    want /= np.linalg.norm(want)
    if want @ w < 0:                                # sign convention: R > 0 keeps w's side
        want = -want
    got = oracle.oja_update(w[:, None], x[None, :], 0.05)[:, 0]
    assert np.max(np.abs(got - want)) < 1e-14


def pin_oja_batch_is_average_of_rows():
    """The batch step is the mean of the single-row steps (before
    orthonormalisation); with r = d the step vanishes (u u^T = I); no rows, no
    change."""
    rng = np.random.default_rng(34)
    u = orthonormal(rng, 24)
    x = rng.standard_normal((5, D))
    eta = 0.01
    mean_step = np.mean([np.outer(xi, xi @ u) - u @ np.outer(xi @ u, xi @ u) for xi in x], axis=0)
    assert np.max(np.abs(oracle.oja_update(u, x, eta) - oracle.orthonormalise(u + eta * mean_step))) < 1e-14
    full = orthonormal(rng, D)
    assert np.max(np.abs(oracle.oja_update(full, x, 0.3) - full)) < 1e-10
    assert np.array_equal(oracle.oja_update(u, np.zeros((0, D)), 0.3), u)


def pin_versions_reduce_and_brute_force():
    """Codes made under two basis versions: equal versions give the one-basis
    decode; distinct versions match brute force on the cache reconstructed
    token by token with each token's own basis, anchors included."""
    rng = np.random.default_rng(35)
    n, w, g, rk, rv = 40, 4, 2, 16, 8
    cpos, apos = oracle.code_positions(n, w), oracle.anchor_positions(n, w)
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, D))
    q = rng.standard_normal((g, D)) * 2
    bk = [orthonormal(rng, rk), orthonormal(rng, rk)]
    bv = [orthonormal(rng, rv), orthonormal(rng, rv)]
    ver = (np.arange(len(cpos)) >= 20).astype(int)
    ck = np.stack([k[j] @ bk[vj] for j, vj in zip(cpos, ver)])
    cv = np.stack([v[j] @ bv[vj] for j, vj in zip(cpos, ver)])
    sc = oracle.default_scale()
    same = oracle.oracle_decode_unit_versions(q, [bk[0], bk[0]], [bv[0], bv[0]], ver,
                                              k[cpos] @ bk[0], v[cpos] @ bv[0], k[apos], v[apos], sc)
    ref = oracle.oracle_decode_unit(q, bk[0], bv[0], k[cpos] @ bk[0], v[cpos] @ bv[0], k[apos], v[apos], sc)
    assert np.max(np.abs(same - ref)) < 1e-12
    got = oracle.oracle_decode_unit_versions(q, bk, bv, ver, ck, cv, k[apos], v[apos], sc)
    khat = np.concatenate([np.stack([bk[vj] @ c for c, vj in zip(ck, ver)]), k[apos]])
    vhat = np.concatenate([np.stack([bv[vj] @ c for c, vj in zip(cv, ver)]), v[apos]])
    for i in range(g):
        want, _ = brute_attention(q[i], khat, vhat, sc)
        assert np.max(np.abs(got[i] - want)) < 1e-12


# ---------------------------------------------------------------------------
# group-head latents
# ---------------------------------------------------------------------------

def pin_group_compress_is_concatenated_projection():
    """The shared code is the sum of each head's rows times its slice (block
    matrix product written out), and a block-diagonal group basis gives each
    head's own per-head codes side by side."""
    rng = np.random.default_rng(36)
    ng, t, r = 3, 7, 24
    x = rng.standard_normal((ng, t, D))
    u = np.linalg.qr(rng.standard_normal((ng * D, ng * D)))[0][:, :r]
    want = sum(x[j] @ u[j * D:(j + 1) * D] for j in range(ng))
    assert np.max(np.abs(oracle.oracle_compress_group(x, u) - want)) < 1e-12
    per = [orthonormal(rng, 8) for _ in range(ng)]
    bd = np.zeros((ng * D, ng * 8))
    for j in range(ng):
        bd[j * D:(j + 1) * D, j * 8:(j + 1) * 8] = per[j]
    got = oracle.oracle_compress_group(x, bd)
    for j in range(ng):
        assert np.max(np.abs(got[:, j * 8:(j + 1) * 8] - x[j] @ per[j])) < 1e-12


def pin_group_decode_brute_force():
    """Each query head of a group against brute force on its own KV head's cache,
    reconstructed token by token from the shared codes with that head's slice;
    with one head per group it is the one-head decode."""
    rng = np.random.default_rng(37)
    ng, g, n, w, rk, rv = 2, 2, 30, 4, 16, 12
    cpos, apos = oracle.code_positions(n, w), oracle.anchor_positions(n, w)
    k = rng.standard_normal((ng, n, D))
    v = rng.standard_normal((ng, n, D))
    uk = np.linalg.qr(rng.standard_normal((ng * D, ng * D)))[0][:, :rk]
    uv = np.linalg.qr(rng.standard_normal((ng * D, ng * D)))[0][:, :rv]
    ck = oracle.oracle_compress_group(k[:, cpos], uk)
    cv = oracle.oracle_compress_group(v[:, cpos], uv)
    q = rng.standard_normal((ng * g, D)) * 2
    heads = np.repeat(np.arange(ng), g)
    sc = oracle.default_scale()
    got = oracle.oracle_decode_group(q, heads, uk, uv, ck, cv, [k[j][apos] for j in range(ng)],
                                     [v[j][apos] for j in range(ng)], sc)
    for i, j in enumerate(heads):
        khat = np.concatenate([reconstruct(ck, uk[j * D:(j + 1) * D]), k[j][apos]])
        vhat = np.concatenate([reconstruct(cv, uv[j * D:(j + 1) * D]), v[j][apos]])
        want, _ = brute_attention(q[i], khat, vhat, sc)
        assert np.max(np.abs(got[i] - want)) < 1e-12
    one = oracle.oracle_decode_group(q[:2], [0, 0], uk[:D], uv[:D], k[0][cpos] @ uk[:D], v[0][cpos] @ uv[:D],
                                     [k[0][apos]], [v[0][apos]], sc)
    ref = oracle.oracle_decode_unit(q[:2], uk[:D], uv[:D], k[0][cpos] @ uk[:D], v[0][cpos] @ uv[:D],
                                    k[0][apos], v[0][apos], sc)
    assert np.max(np.abs(one - ref)) < 1e-12


def pin_lowram_fit_recovers_map_and_matches_lstsq():
    """Values that are an exact linear map of the codes give that map back; on
    general rows the fit equals NumPy's least-squares solver on the ridge-augmented
    system [C; sqrt(lam) I] M = [V; 0] (lam = 1e-6 tr(C^T C) / r)."""
    rng = np.random.default_rng(40)
    t, r = 300, 16
    c = rng.standard_normal((t, r)) * np.exp(-np.arange(r) / 8)
    a = rng.standard_normal((r, D))
    got = oracle.lowram_fit(c, c @ a)
    assert np.max(np.abs(got - a)) < 1e-3 * np.max(np.abs(a)), np.max(np.abs(got - a))
    v = rng.standard_normal((t, D)) + c @ a
    lam = 1e-6 * np.sum(c * c) / r
    aug_c = np.concatenate([c, math.sqrt(lam) * np.eye(r)])
    aug_v = np.concatenate([v, np.zeros((r, D))])
    want = np.linalg.lstsq(aug_c, aug_v, rcond=None)[0]
    assert np.max(np.abs(oracle.lowram_fit(c, v) - want)) < 1e-9 * np.max(np.abs(want))
    # an all-zero code matrix predicts nothing
    assert not np.any(oracle.lowram_fit(np.zeros((5, r)), rng.standard_normal((5, D))))


def pin_lowram_select_is_blockwise_top_r():
    """Per block of 32 slots, exactly min(r, block size) slots are kept, and every
    kept slot's norm beats every dropped slot's (equal norms: the lower slot is
    kept); the same set comes out of inserting the slots one at a time in slot
    order into a set of at most r, replacing the smallest only when strictly
    beaten (the decode-time rule)."""
    rng = np.random.default_rng(41)
    for n, r in ((77, 5), (32, 1), (40, 32), (10, 3), (64, 8)):
        sq = rng.integers(0, 6, n).astype(float)        # many ties
        kept = set(oracle.lowram_select(sq, r).tolist())
        for b0 in range(0, n, 32):
            blk = list(range(b0, min(b0 + 32, n)))
            k = [j for j in blk if j in kept]
            d = [j for j in blk if j not in kept]
            assert len(k) == min(r, len(blk))
            for i in k:
                for j in d:
                    assert sq[i] > sq[j] or (sq[i] == sq[j] and i < j), (n, r, i, j)
            online = []
            for j in blk:
                if len(online) < r:
                    online.append(j)
                else:
                    low = min(online, key=lambda x: (sq[x], -x))
                    if sq[j] > sq[low]:
                        online[online.index(low)] = j
            assert sorted(online) == k, (n, r)


def pin_lowram_decode_brute_force():
    """Brute force over the reconstructed cache: keys U_K c_t, values M^T c_t plus
    the residual of kept slots, anchors at full rank.  With every residual kept and
    unrounded the values are the original rows."""
    rng = np.random.default_rng(42)
    n, w, rk, g = 45, 4, 16, 3
    cpos, apos = oracle.code_positions(n, w), oracle.anchor_positions(n, w)
    k = rng.standard_normal((n, D))
    v = rng.standard_normal((n, D)) * 0.5 + k @ rng.standard_normal((D, D)) * 0.05
    uk = orthonormal(rng, rk)
    ck = k[cpos] @ uk
    q = rng.standard_normal((g, D)) * 3
    sc = oracle.default_scale()
    m, kept, e = oracle.lowram_prefill(ck, v[cpos], 5)
    got = oracle.oracle_decode_lowram(q, uk, m, ck, kept, e, k[apos], v[apos], sc)
    keys = np.concatenate([reconstruct(ck, uk), k[apos]])
    vals = [np.asarray(m, float).T @ ck[t] + (e[t] if t in set(kept.tolist()) else 0) for t in range(len(cpos))]
    vals = np.concatenate([np.stack(vals), v[apos]])
    for i in range(g):
        want, _ = brute_attention(q[i], keys, vals, sc)
        assert np.max(np.abs(got[i] - want)) < 1e-12
    exact_e = oracle.lowram_residuals(ck, v[cpos], m)
    full = oracle.oracle_decode_lowram(q, uk, m, ck, np.arange(len(cpos)), exact_e, k[apos], v[apos], sc)
    for i in range(g):
        want, _ = brute_attention(q[i], keys, np.concatenate([v[cpos], v[apos]]), sc)
        assert np.max(np.abs(full[i] - want)) < 1e-12


def pin_rope_is_the_complex_rotation():
    """RoPE against its complex form, (x_i + i x_(i+64)) e^(i p theta_i) with
    theta_i = base^(-i/64) written out per pair; identity at position 0; norms
    kept; dot products depend only on the position difference; p then -p is the
    identity."""
    rng = np.random.default_rng(50)
    base = 10000.0
    x = rng.standard_normal((5, D))
    pos = np.array([0, 1, 7, 1000, 32767])
    got = oracle.rope(x, pos, base)
    for r in range(5):
        for i in range(D // 2):
            z = complex(x[r, i], x[r, i + 64]) * complex(math.cos(pos[r] * base ** (-i / 64)),
                                                          math.sin(pos[r] * base ** (-i / 64)))
            assert abs(got[r, i] - z.real) < 1e-9 and abs(got[r, i + 64] - z.imag) < 1e-9, (r, i)
    assert np.array_equal(oracle.rope(x[:1], [0], base), x[:1])
    assert np.allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    q, k = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    d1 = float((oracle.rope(q, [100], base) @ oracle.rope(k, [40], base).T)[0, 0])
    d2 = float((oracle.rope(q, [5060], base) @ oracle.rope(k, [5000], base).T)[0, 0])
    assert abs(d1 - d2) < 1e-9
    assert np.allclose(oracle.rope(oracle.rope(x, pos, base), -pos, base), x, atol=1e-9)


def pin_prerope_decode_brute_force():
    """Brute force: every compressed key reconstructed token by token from its
    code, rotated to its position as a complex number per pair, then softmax
    attention with loops; at position 0 everywhere it is the code-space decode."""
    rng = np.random.default_rng(51)
    n, w, rk, rv, g, base = 40, 4, 16, 16, 2, 500000.0
    cpos, apos = oracle.code_positions(n, w), oracle.anchor_positions(n, w)
    k_pre = rng.standard_normal((n, D))
    v = rng.standard_normal((n, D))
    uk, uv = orthonormal(rng, rk), orthonormal(rng, rv)
    ck, cv = k_pre[cpos] @ uk, v[cpos] @ uv
    q = rng.standard_normal((g, D)) * 2
    k_a = oracle.rope(k_pre[apos], apos, base)
    sc = oracle.default_scale()
    got = oracle.oracle_decode_unit_prerope(q, uk, uv, ck, cv, cpos, k_a, v[apos], sc, base)
    keys = []
    for t, p in enumerate(cpos):
        kh = uk @ ck[t]
        rot = np.empty(D)
        for i in range(D // 2):
            z = complex(kh[i], kh[i + 64]) * complex(math.cos(p * base ** (-i / 64)), math.sin(p * base ** (-i / 64)))
            rot[i], rot[i + 64] = z.real, z.imag
        keys.append(rot)
    keys = np.concatenate([np.stack(keys), k_a])
    vals = np.concatenate([reconstruct(cv, uv), v[apos]])
    for i in range(g):
        want, _ = brute_attention(q[i], keys, vals, sc)
        assert np.max(np.abs(got[i] - want)) < 1e-12
    zero = oracle.oracle_decode_unit_prerope(q, uk, uv, ck, cv, np.zeros(len(cpos)), k_pre[apos], v[apos], sc, base)
    ref = oracle.oracle_decode_unit(q, uk, uv, ck, cv, k_pre[apos], v[apos], sc)
    assert np.max(np.abs(zero - ref)) < 1e-12


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
