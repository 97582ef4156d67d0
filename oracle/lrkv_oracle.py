"""CPU oracle for decode attention read directly from a low-rank-compressed KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports this module; only the
test suite, the smoke check and the CPU-baseline leg of the benchmark call it.
It shares no code, tables or helpers with the HIP path.

Everything is float64 NumPy, written for a reader to check against the pages by
eye; there is no blocking, fusion or reordering beyond what the definition needs.

What it follows:

* "Half the Memory, None of the Answers Lost" (altslate blog), section 04 "what
  worked": one projection per (layer, head) maps each 128-dim key (taken after
  RoPE) and value to an r-dim code, r < 128; the codes are what is stored.
* The same blog, section 08 "at serving time": attention can be computed against
  the codes themselves, which is algebraically the same as reconstructing the
  cache; the projection matrices are shared per head.
* "OjaKV: Online Low-Rank Compression for LLM Key-Value Caches" (astrobobo
  article), FAQ on which tokens are compressed: the first token and the most
  recent tokens are kept at full rank as anchors; every token in between is
  stored low-rank.

Readings where the pages are silent (each also listed in the design doc):

* the score scale is 1/sqrt(d) with d = 128, the model's own scale;
* ``n`` counts the cached tokens including the decode token itself; the anchor
  set is {0} plus the last ``window`` tokens, the codes are everything between;
* query head i of a GQA group reads KV head i // g;
* codes are ``x @ U`` with U a (128, r) matrix with orthonormal columns.

Group-head latents (Palu's medium-grained decomposition) share one code stream
among the KV heads of a group, each head reading its own slice of the group
basis; see oracle_compress_group and oracle_decode_group.

Online basis adaptation (OjaKV) uses the textbook Oja subspace rule with
re-orthonormalisation (the page names Oja's algorithm but gives no rule); codes
made under several basis versions are decoded each with its own version; see
oja_update and oracle_decode_unit_versions.

Keys compressed before RoPE (Palu) are reconstructed and rotated per token
before scoring (standard rotate-half RoPE); see oracle_decode_unit_prerope.

LowRAM's value amortisation (values predicted from the key codes by a linear
map fitted on the prompt, residuals kept for each block's worst-predicted tokens)
follows readings stated with lowram_fit; see oracle_decode_lowram.

Int8 and int4 codes (the first step past the pages: they name quantisation of
the low-rank cache but no quantiser) follow a stated design, symmetric with one
float32 scale per code row, decided in float32; see quantize_codes_q8 and
quantize_codes_q4.

Pins (tests/test_oracle.py): full attention at r = d with an orthogonal basis
(the blog's section 04 plumbing check), brute-force reconstruction on tiny
inputs, torch's float64 scaled_dot_product_attention, softmax weights summing to
one, closed forms (n = 1, q = 0, constant values), invariances (basis sign, token
order), compress closed forms and the OjaKV FAQ's ~16 GB KV-cache size; the Oja
step against eigendecomposition fixed points, the LowRAM fit against least
squares, pre-RoPE decode against the complex-rotation form, group latents
against block products (tests/oracle_pins.py, with planted mistakes in
tests/test_oracle_mutants.py).  Every function here has such a pin; the pages
print no worked example of the decode, so no pin is a printed value except the
cache size.
"""

from __future__ import annotations

import math

import numpy as np

HEAD_DIM = 128


# ---------------------------------------------------------------------------
# number format
# ---------------------------------------------------------------------------

def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 value, ties to even, straight from float64.

    bfloat16 keeps 8 significant bits (7 stored) and float32's exponent range;
    below the smallest normal (2**-126) the spacing stays 2**-133.  Written from
    that definition: quantum = 2**(e - 8) for a frexp exponent e (mantissa in
    [0.5, 1)), and np.rint rounds half to even.  Overflow is not handled (the
    workloads never come near it)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    quantum = np.ldexp(1.0, e - 8)
    return np.rint(x / quantum) * quantum


# ---------------------------------------------------------------------------
# which tokens are anchors (OjaKV FAQ), which are codes (blog section 04)
# ---------------------------------------------------------------------------

def anchor_positions(n: int, window: int) -> np.ndarray:
    """Token 0 plus the most recent ``window`` tokens, kept at full rank."""
    if n < 1:
        raise ValueError("n must be >= 1")
    recent = range(max(1, n - window), n)
    return np.array([0, *recent], dtype=np.int64)


def code_positions(n: int, window: int) -> np.ndarray:
    """Tokens strictly between the first token and the recent window."""
    return np.arange(1, max(1, n - window), dtype=np.int64)


# ---------------------------------------------------------------------------
# prefill compression (blog section 04)
# ---------------------------------------------------------------------------

def oracle_compress(x, u) -> np.ndarray:
    """Codes of the rows of ``x`` (t, 128) under the basis ``u`` (128, r): x @ u."""
    x = np.asarray(x, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    return x @ u


# ---------------------------------------------------------------------------
# decode attention against codes and anchors (blog section 08), one step at a time
# ---------------------------------------------------------------------------

def project_query(q, u_k) -> np.ndarray:
    """q~ = U_K^T q for each query row: (g, 128) -> (g, r_k)."""
    return np.asarray(q, np.float64) @ np.asarray(u_k, np.float64)


def code_scores(q_tilde, c_k, scale: float) -> np.ndarray:
    """Scores of the compressed tokens, taken in code space: (g, c)."""
    return (q_tilde @ np.asarray(c_k, np.float64).T) * scale


def anchor_scores(q, k_a, scale: float) -> np.ndarray:
    """Scores of the full-rank anchor tokens: (g, a)."""
    return (np.asarray(q, np.float64) @ np.asarray(k_a, np.float64).T) * scale


def softmax_weights(s) -> tuple:
    """One softmax over all scores of a query row.  Returns the unnormalised
    weights e = exp(s - max s) and their sum L (so p = e / L)."""
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e, e.sum(axis=1, keepdims=True)


def rank_space_values(e_codes, c_v) -> np.ndarray:
    """o~ = sum_j e_j c^V_j, accumulated in the r_v-dim code space: (g, r_v)."""
    return e_codes @ np.asarray(c_v, np.float64)


def anchor_values(e_anchors, v_a) -> np.ndarray:
    """sum_j e_j v_j over the anchors, in full 128-dim space: (g, 128)."""
    return e_anchors @ np.asarray(v_a, np.float64)


def up_project(o_tilde, u_v) -> np.ndarray:
    """The single up-projection U_V o~ per query row: (g, r_v) -> (g, 128)."""
    return o_tilde @ np.asarray(u_v, np.float64).T


def oracle_decode_unit(q, u_k, u_v, c_k, c_v, k_a, v_a, scale: float, return_p: bool = False):
    """Decode attention of the g query heads that share one KV head.

    q (g, 128); u_k (128, r_k); u_v (128, r_v); c_k (c, r_k); c_v (c, r_v);
    k_a, v_a (a, 128).  Returns out (g, 128) and, if asked, the normalised
    weights p (g, c + a) with the code tokens first, then the anchors."""
    c = np.asarray(c_k).shape[0]
    q_tilde = project_query(q, u_k)
    s = np.concatenate([code_scores(q_tilde, c_k, scale), anchor_scores(q, k_a, scale)], axis=1)
    e, total = softmax_weights(s)
    o_tilde = rank_space_values(e[:, :c], c_v)
    out = (up_project(o_tilde, u_v) + anchor_values(e[:, c:], v_a)) / total
    if return_p:
        return out, e / total
    return out


def default_scale(d: int = HEAD_DIM) -> float:
    return 1.0 / math.sqrt(d)


def oracle_decode_layer(q, bases_k, bases_v, codes_k, codes_v, anchors_k, anchors_v,
                        scale: float | None = None) -> np.ndarray:
    """One decode step of a whole layer.

    q (batch, Hq, 128); bases_k[h] (128, r_k[h]); bases_v[h] (128, r_v[h]);
    codes_k[b][h] (c_b, r_k[h]); codes_v[b][h] (c_b, r_v[h]);
    anchors_k[b][h], anchors_v[b][h] (a_b, 128).  Query head i reads KV head
    i // g.  Returns out (batch, Hq, 128) in float64."""
    q = np.asarray(q, np.float64)
    batch, n_q, _ = q.shape
    n_kv = len(bases_k)
    g = n_q // n_kv
    scale = default_scale() if scale is None else scale
    out = np.empty((batch, n_q, HEAD_DIM))
    for b in range(batch):
        for h in range(n_kv):
            rows = slice(h * g, (h + 1) * g)
            out[b, rows] = oracle_decode_unit(
                q[b, rows], bases_k[h], bases_v[h], codes_k[b][h], codes_v[b][h],
                anchors_k[b][h], anchors_v[b][h], scale)
    return out


# ---------------------------------------------------------------------------
# online subspace adaptation (OjaKV summary and FAQ: Oja's algorithm for online
# PCA keeps adapting the projection basis, thoroughly during prompt prefill and
# lightly, now and then, during decoding; older codes stay in the basis they were
# made with).  The page names the algorithm but prints no update rule, step size
# or schedule, so the textbook subspace rule is used, with the columns brought
# back to orthonormal after every step (the decode reads bases as orthonormal).
# ---------------------------------------------------------------------------

def orthonormalise(a) -> np.ndarray:
    """The Q of the thin QR factorisation of ``a`` (d, r) whose R has a positive
    diagonal: the columns Gram-Schmidt gives, in order.  Columns must be
    linearly independent."""
    a = np.asarray(a, np.float64)
    q, r = np.linalg.qr(a)
    return q * np.sign(np.diag(r))[None, :]


def oja_update(u, x, eta: float) -> np.ndarray:
    """One step of Oja's subspace rule on a batch of rows.

    u (d, r) with orthonormal columns; x (N, d): the rows seen since the last
    step (keys after RoPE, or values); eta: the step size.  With y = x u (the
    rows' codes), u' = u + eta (x^T y - u y^T y) / N, i.e. the rule's average
    over the batch; then u' is orthonormalised.  N = 0 leaves u unchanged."""
    u = np.asarray(u, np.float64)
    x = np.asarray(x, np.float64)
    n = x.shape[0]
    if n == 0:
        return u.copy()
    y = x @ u
    grad = (x.T @ y - u @ (y.T @ y)) / n
    return orthonormalise(u + eta * grad)


def oracle_decode_unit_versions(q, bases_k, bases_v, versions, c_k, c_v, k_a, v_a,
                                scale: float) -> np.ndarray:
    """Decode attention of one GQA group when its code tokens were made under
    several bases: code token j was compressed with bases_k[versions[j]] and
    bases_v[versions[j]].  Each token is scored against the query projected
    with its own key basis and its value sum is up-projected with its own value
    basis; one softmax covers every code token and the anchors.  Returns out
    (g, 128)."""
    q = np.asarray(q, np.float64)
    versions = np.asarray(versions, np.int64)
    c_k = np.asarray(c_k, np.float64)
    c_v = np.asarray(c_v, np.float64)
    c = len(versions)
    s_codes = np.zeros((q.shape[0], c))
    for v in np.unique(versions):
        sel = versions == v
        s_codes[:, sel] = code_scores(project_query(q, bases_k[v]), c_k[sel], scale)
    s = np.concatenate([s_codes, anchor_scores(q, k_a, scale)], axis=1)
    e, total = softmax_weights(s)
    out = anchor_values(e[:, c:], v_a)
    for v in np.unique(versions):
        sel = versions == v
        out = out + up_project(rank_space_values(e[:, :c][:, sel], c_v[sel]), bases_v[v])
    return out / total


# ---------------------------------------------------------------------------
# group-head latents (Palu abstract: a medium-grained low-rank decomposition
# between one latent per head and one for all heads).  Reading: the n_g KV heads
# of a group share one code per token, the projection of their concatenated
# keys (values) onto one (n_g * 128, r) basis with orthonormal columns; KV head
# j of the group reconstructs as its 128-row slice of the basis times the code.
# ---------------------------------------------------------------------------

def oracle_compress_group(x_heads, u_group) -> np.ndarray:
    """Shared codes of a head group: x_heads (n_g, t, 128) the group's rows (head
    by head), u_group (n_g * 128, r).  Returns (t, r): [x_1 ... x_ng] u_group."""
    x = np.asarray(x_heads, np.float64)
    joined = np.concatenate(list(x), axis=1)  # (t, n_g * 128), head 0's features first
    return joined @ np.asarray(u_group, np.float64)


def group_slice(u_group, j: int) -> np.ndarray:
    """KV head j's (128, r) slice of a group basis: rows 128 j .. 128 j + 127."""
    return np.asarray(u_group, np.float64)[HEAD_DIM * j:HEAD_DIM * (j + 1)]


def oracle_decode_group(q, head_of_query, u_k_group, u_v_group, c_k, c_v, k_a, v_a,
                        scale: float) -> np.ndarray:
    """Decode attention of the query heads of one head group against its shared
    codes.  q (m, 128); head_of_query (m,) the group-local KV head j of each
    query; u_k_group (n_g * 128, r_k), u_v_group (n_g * 128, r_v); c_k (c, r_k),
    c_v (c, r_v) shared; k_a[j], v_a[j] (a, 128) the anchors of KV head j.
    Query i is the one-head decode with KV head j's slices of the bases, the
    shared codes and KV head j's anchors.  Returns out (m, 128)."""
    q = np.asarray(q, np.float64)
    out = np.empty((q.shape[0], HEAD_DIM))
    for i, j in enumerate(head_of_query):
        out[i] = oracle_decode_unit(q[i:i + 1], group_slice(u_k_group, j), group_slice(u_v_group, j),
                                    c_k, c_v, k_a[j], v_a[j], scale)[0]
    return out


# ---------------------------------------------------------------------------
# int8 codes with one scale per token.  The pages pair low-rank caches with
# quantisation (LowRAM abstract: the method composes with quantisation; Palu
# abstract: low-rank-aware quantisation) but print no quantiser, so this one is
# a design choice: symmetric, one scale per (token, head, K or V), decided in
# float32 so that both sides take the same integer decisions.
# ---------------------------------------------------------------------------

def quantize_codes_q8(x32) -> tuple:
    """Quantise code rows ``x32`` (t, r), given as float32, to int8.

    Per row, all in float32: a = max |x|; s = a / 127 (rounded to nearest even);
    q = x / s rounded to nearest, ties to even, clipped to [-127, 127].  A row of
    zeros gets s = 0 and q = 0.  Returns (q int8 (t, r), s float32 (t,))."""
    x = np.asarray(x32, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x32 must be (t, r)")
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (a / np.float32(127)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    q = np.rint(x / safe[:, None])
    q = np.clip(q, -127, 127)
    q[s == 0] = 0
    return q.astype(np.int8), s


def dequantize_codes_q8(q, s) -> np.ndarray:
    """The codes an int8 row stands for: s * q, exact in float64."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[:, None]


def quantize_codes_q4(x32) -> tuple:
    """Quantise code rows ``x32`` (t, r), given as float32, to 4-bit integers.

    The int8 rule with 7 in place of 127: per row, in float32, a = max |x|,
    s = a / 7, q = x / s rounded to nearest, ties to even, clipped to [-7, 7]; a
    row of zeros gets s = 0 and q = 0.  Returns (q int8 holding values in [-7, 7]
    (t, r), s float32 (t,))."""
    x = np.asarray(x32, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("x32 must be (t, r)")
    a = np.max(np.abs(x), axis=1) if x.shape[1] else np.zeros(x.shape[0], np.float32)
    s = (a / np.float32(7)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    q = np.rint(x / safe[:, None])
    q = np.clip(q, -7, 7)
    q[s == 0] = 0
    return q.astype(np.int8), s


def dequantize_codes_q4(q, s) -> np.ndarray:
    """The codes a 4-bit row stands for: s * q, exact in float64."""
    return np.asarray(q, np.float64) * np.asarray(s, np.float64)[:, None]


# ---------------------------------------------------------------------------
# byte accounting (OjaKV FAQ: ~16 GB of KV for Llama-3.1-8B, 32K tokens, batch 4;
# blog section 08: the per-request cache shrinks with the code width, plus the
# shared projection matrices)
# ---------------------------------------------------------------------------

# ---------------------------------------------------------------------------
# LowRAM value amortisation (LowRAM abstract: inside one attention head the
# values are largely predictable from their keys; a light per-head predictor is
# fitted at test time and residuals are stored only for the tokens it
# reconstructs worst).  The page fixes neither the predictor nor the selection
# rule; the readings (also in the design doc):
#   * the predictor is linear in the stored key codes, V ~ C_K M with M of shape
#     (r_k, 128), one per (batch row, KV head), fitted on the prompt's compressed
#     tokens by least squares with a tiny relative ridge for rank-deficient code
#     matrices: M = (C_K^T C_K + lam I)^-1 C_K^T V, lam = 1e-6 tr(C_K^T C_K) / r_k;
#   * the residual of a token is e_t = V_t - C_K,t M with M as stored (bf16);
#     every 32-slot block keeps the residuals of its R tokens with the largest
#     squared norm (ties: the lower slot), stored in bf16;
#   * the decode reads value C_K,t M + e_t for a kept token, C_K,t M otherwise.
# ---------------------------------------------------------------------------

LOWRAM_BLOCK = 32
LOWRAM_RIDGE = 1e-6


def lowram_fit(c_k, v) -> np.ndarray:
    """Predictor M (r_k, 128) of values from key codes: ridge-stabilised least
    squares over the rows of c_k (t, r_k) and v (t, 128)."""
    c = np.asarray(c_k, np.float64)
    x = np.asarray(v, np.float64)
    a = c.T @ c
    lam = LOWRAM_RIDGE * np.trace(a) / a.shape[0] + 1e-30
    return np.linalg.solve(a + lam * np.eye(a.shape[0]), c.T @ x)


def lowram_residuals(c_k, v, m) -> np.ndarray:
    """e_t = v_t - c_t M for every row."""
    return np.asarray(v, np.float64) - np.asarray(c_k, np.float64) @ np.asarray(m, np.float64)


def lowram_select(sq_norms, r: int) -> np.ndarray:
    """Slots whose residual is kept: in every block of 32 consecutive slots, the r
    with the largest squared norm (ties: the lower slot).  Sorted slot indices."""
    sq = np.asarray(sq_norms, np.float64)
    kept = []
    for b0 in range(0, len(sq), LOWRAM_BLOCK):
        block = list(range(b0, min(b0 + LOWRAM_BLOCK, len(sq))))
        block.sort(key=lambda j: (-sq[j], j))
        kept += block[:r]
    return np.array(sorted(kept), dtype=np.int64)


def lowram_prefill(c_k, v, r: int) -> tuple:
    """What a prompt leaves in the cache: (M as stored (bf16), kept slots, the
    residual rows of every slot as stored (bf16)); only the kept rows are read."""
    m = bf16_round(lowram_fit(c_k, v))
    e = lowram_residuals(c_k, v, m)
    kept = lowram_select(np.sum(e * e, axis=1), r)
    return m, kept, bf16_round(e)


def lowram_values(c_k, m, kept, e) -> np.ndarray:
    """The values the decode reads for the compressed tokens: C_K M, plus the
    residual rows of the kept slots."""
    vals = np.asarray(c_k, np.float64) @ np.asarray(m, np.float64)
    kept = np.asarray(kept, np.int64)
    vals[kept] += np.asarray(e, np.float64)[kept]
    return vals


def oracle_decode_lowram(q, u_k, m, c_k, kept, e, k_a, v_a, scale: float) -> np.ndarray:
    """Decode attention of the g query heads of one KV head over a LowRAM cache:
    keys as in oracle_decode_unit (scored against the codes), values of the
    compressed tokens from lowram_values, anchors at full rank.  q (g, 128),
    u_k (128, r_k), m (r_k, 128), c_k (c, r_k), kept (slots), e (c, 128),
    k_a, v_a (a, 128).  Returns out (g, 128)."""
    vals = lowram_values(c_k, m, kept, e)
    return oracle_decode_unit(q, u_k, np.eye(HEAD_DIM), c_k, vals, k_a, v_a, scale)


# ---------------------------------------------------------------------------
# Keys compressed before RoPE (Palu abstract: the full keys and values are
# reconstructed on the fly; a decomposition of the key projection keeps the
# latents before the rotary position embedding, so the keys cannot be scored in
# code space any more).  The rotation is the standard rotate-half RoPE (the pages
# name RoPE but print no formula): feature pair (i, i + 64), i < 64, of a key or
# query at position p turns by the angle p * base^(-2 i / 128).  Codes hold the
# pre-RoPE keys' projections; anchors and the query are post-RoPE, as attention
# uses them; values are never rotated.
# ---------------------------------------------------------------------------

def rope(x, positions, base: float) -> np.ndarray:
    """Rotate-half RoPE of rows x (t, 128) at the given positions (t,)."""
    x = np.asarray(x, np.float64)
    half = HEAD_DIM // 2
    theta = float(base) ** (-2.0 * np.arange(half) / HEAD_DIM)
    ang = np.asarray(positions, np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=1)


def oracle_decode_unit_prerope(q, u_k, u_v, c_k, c_v, code_pos, k_a, v_a, scale: float,
                               base: float) -> np.ndarray:
    """Decode attention over codes of pre-RoPE keys: each compressed key is
    reconstructed (U_K c_t) and rotated to its position code_pos[t], then scored
    with the post-RoPE query q (g, 128); anchors k_a are post-RoPE; values stay
    in code space (one up-projection).  Returns out (g, 128)."""
    c = np.asarray(c_k).shape[0]
    keys = rope(np.asarray(c_k, np.float64) @ np.asarray(u_k, np.float64).T, code_pos, base)
    q = np.asarray(q, np.float64)
    s = np.concatenate([scale * (q @ keys.T), anchor_scores(q, k_a, scale)], axis=1)
    e, total = softmax_weights(s)
    return (up_project(rank_space_values(e[:, :c], c_v), u_v) + anchor_values(e[:, c:], v_a)) / total


def full_kv_bytes(n_layers: int, n_kv_heads: int, n_tokens: int, batch: int,
                  head_dim: int = HEAD_DIM, elem_bytes: int = 2) -> int:
    """Bytes of an uncompressed cache: keys and values of every layer and KV head."""
    return 2 * n_layers * n_kv_heads * head_dim * n_tokens * batch * elem_bytes


def compressed_unit_bytes(n: int, window: int, r_k: int, r_v: int, elem_bytes: int = 2,
                          head_dim: int = HEAD_DIM, q8: bool = False, q4: bool = False) -> int:
    """Bytes one decode step must read for one (batch row, KV head): the codes of
    the compressed tokens plus the full-rank anchors.  With int8 codes each code
    row is r bytes plus its 4-byte scale, with 4-bit codes r / 2 bytes plus the
    scale; anchors stay at ``elem_bytes``."""
    c = len(code_positions(n, window))
    a = len(anchor_positions(n, window))
    if q4:
        code_bytes = (r_k + r_v) // 2 + 8
    else:
        code_bytes = (r_k + r_v + 8) if q8 else (r_k + r_v) * elem_bytes
    return c * code_bytes + a * 2 * head_dim * elem_bytes
