"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  A mutant survives only if every pin still passes."""

import numpy as np
import pytest

import oracle
import oracle.lrkv_oracle as lo
import oracle_pins


def _any_pin_fails():
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except Exception:  # AssertionError or a shape error both count as caught
            return True
    return False


def _two_softmaxes(q, u_k, u_v, c_k, c_v, k_a, v_a, scale, return_p=False):
    c = np.asarray(c_k).shape[0]
    qt = lo.project_query(q, u_k)
    out = 0
    for s, vals in [(lo.code_scores(qt, c_k, scale), None), (lo.anchor_scores(q, k_a, scale), v_a)]:
        if s.shape[1] == 0:
            continue
        e, tot = lo.softmax_weights(s)
        part = lo.up_project(lo.rank_space_values(e, c_v), u_v) if vals is None else lo.anchor_values(e, vals)
        out = out + part / tot
    return (out, None) if return_p else out


MUTANTS = {
    "scale_by_rank": ("code_scores", lambda qt, ck, scale: (qt @ np.asarray(ck, float).T) / np.sqrt(np.asarray(ck).shape[1])),
    "anchor_values_dropped": ("anchor_values", lambda e, v: np.zeros((e.shape[0], 128))),
    "up_projection_transposed": ("up_project", lambda o, u: o @ np.asarray(u, float)),
    "query_not_projected": ("project_query", lambda q, u: np.asarray(q, float)[:, : np.asarray(u).shape[1]]),
    "anchor_window_off_by_one": ("anchor_positions", lambda n, w: np.array([0, *range(max(1, n - w - 1), n)])),
    "codes_include_window_edge": ("code_positions", lambda n, w: np.arange(1, max(1, n - w + 1))),
    "bf16_truncates": ("bf16_round", lambda x: np.asarray(np.asarray(x, np.float32).view(np.uint32) & 0xFFFF0000, np.uint32).view(np.float32).astype(np.float64)),
    "no_normalisation": ("softmax_weights", lambda s: (np.exp(s - s.max(axis=1, keepdims=True)), np.ones((s.shape[0], 1)))),
    "values_through_key_basis": ("up_project", None),
    "two_separate_softmaxes": ("oracle_decode_unit", _two_softmaxes),
    "gqa_modulo_mapping": ("oracle_decode_layer", None),
    "missing_scale": ("anchor_scores", lambda q, ka, scale: np.asarray(q, float) @ np.asarray(ka, float).T),
    "q8_ties_away_from_zero": ("quantize_codes_q8", lambda x: _q8_variant(x, rounding="away")),
    "q8_scale_over_128": ("quantize_codes_q8", lambda x: _q8_variant(x, divisor=128)),
    "q8_divisor_127_5": ("quantize_codes_q8", lambda x: _q8_variant(x, divisor=127.5)),
    "q4_ties_away_from_zero": ("quantize_codes_q4", lambda x: _q8_variant(x, rounding="away", divisor=7, qmax=7)),
    "q4_scale_over_8": ("quantize_codes_q4", lambda x: _q8_variant(x, divisor=8, qmax=7)),
    "q4_clip_at_8": ("quantize_codes_q4", lambda x: _q8_variant(x, divisor=7.5, qmax=8)),
    "oja_decay_term_sign": ("oja_update", lambda u, x, eta: _oja_variant(u, x, eta, sign=+1)),
    "oja_not_averaged": ("oja_update", lambda u, x, eta: _oja_variant(u, x, eta, average=False)),
    "oja_not_orthonormalised": ("oja_update", lambda u, x, eta: _oja_variant(u, x, eta, orth=False)),
    "oja_gram_schmidt_reversed": ("oja_update", lambda u, x, eta: _oja_variant(u, x, eta, reverse=True)),
    "versions_one_key_basis": ("oracle_decode_unit_versions", lambda *a: _versions_variant(*a, key_v0=True)),
    "versions_one_value_basis": ("oracle_decode_unit_versions", lambda *a: _versions_variant(*a, val_v0=True)),
    "group_heads_reversed": ("oracle_compress_group",
                             lambda x, u: np.concatenate(list(np.asarray(x, float))[::-1], axis=1) @ np.asarray(u, float)),
    "lowram_residual_sign": ("lowram_values", lambda c, m, kept, e: _lowram_values_variant(c, m, kept, e, sign=-1)),
    "lowram_residual_dropped": ("lowram_values", lambda c, m, kept, e: _lowram_values_variant(c, m, [], e)),
    "lowram_fit_diagonal": ("lowram_fit", lambda c, v: np.asarray(c, float).T @ np.asarray(v, float)
                            / np.maximum(np.sum(np.asarray(c, float) ** 2, axis=0), 1e-30)[:, None]),
    "lowram_fit_no_ridge_scale": ("lowram_fit", lambda c, v: np.linalg.solve(
        np.asarray(c, float).T @ np.asarray(c, float) + 1e-2 * np.eye(np.asarray(c).shape[1]),
        np.asarray(c, float).T @ np.asarray(v, float))),
    "lowram_select_smallest": ("lowram_select", lambda sq, r: _lowram_select_variant(sq, r, sign=-1)),
    "lowram_select_ties_high_slot": ("lowram_select", lambda sq, r: _lowram_select_variant(sq, r, tie=-1)),
    "lowram_select_whole_row": ("lowram_select", lambda sq, r: _lowram_select_variant(sq, r, block=10 ** 9)),
    "rope_interleaved_pairs": ("rope", lambda x, pos, base: _rope_variant(x, pos, base, interleaved=True)),
    "rope_sin_sign": ("rope", lambda x, pos, base: _rope_variant(x, pos, base, sign=-1)),
    "rope_theta_exponent": ("rope", lambda x, pos, base: _rope_variant(x, pos, base, expo=1.0)),
    "prerope_positions_off_by_one": ("oracle_decode_unit_prerope",
                                     lambda q, uk, uv, ck, cv, pos, ka, va, sc, base:
                                     _ORIG_PREROPE(q, uk, uv, ck, cv, np.asarray(pos) + 1, ka, va, sc, base)),
    "group_slice_off_by_one_head": ("group_slice", lambda u, j: np.asarray(u, float)[128 * max(j - 1, 0):128 * max(j, 1)]),
}


def _rope_variant(x, pos, base, interleaved=False, sign=1, expo=2.0):
    x = np.asarray(x, float)
    theta = float(base) ** (-expo * np.arange(64) / 128)
    ang = np.asarray(pos, float)[:, None] * theta[None, :]
    c, s = np.cos(ang), sign * np.sin(ang)
    if interleaved:
        a, b = x[:, 0::2], x[:, 1::2]
        out = np.empty_like(x)
        out[:, 0::2], out[:, 1::2] = a * c - b * s, a * s + b * c
        return out
    a, b = x[:, :64], x[:, 64:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=1)


_ORIG_PREROPE = lo.oracle_decode_unit_prerope


def _lowram_values_variant(c, m, kept, e, sign=1):
    vals = np.asarray(c, float) @ np.asarray(m, float)
    kept = np.asarray(kept, np.int64)
    vals[kept] += sign * np.asarray(e, float)[kept]
    return vals


def _lowram_select_variant(sq, r, sign=1, tie=1, block=32):
    sq = np.asarray(sq, float)
    kept = []
    for b0 in range(0, len(sq), block):
        blk = sorted(range(b0, min(b0 + block, len(sq))), key=lambda j: (-sign * sq[j], tie * j))
        kept += blk[:r]
    return np.array(sorted(kept), dtype=np.int64)


def _oja_variant(u, x, eta, sign=-1, average=True, orth=True, reverse=False):
    u = np.asarray(u, float)
    x = np.asarray(x, float)
    if len(x) == 0:
        return u.copy()
    y = x @ u
    step = x.T @ y + sign * (u @ (y.T @ y))
    if average:
        step = step / len(x)
    a = u + eta * step
    if not orth:
        return a
    if reverse:
        return lo.orthonormalise(a[:, ::-1])[:, ::-1]
    return lo.orthonormalise(a)


def _versions_variant(q, bases_k, bases_v, versions, c_k, c_v, k_a, v_a, scale, key_v0=False, val_v0=False):
    bk = [bases_k[0]] * len(bases_k) if key_v0 else bases_k
    bv = [bases_v[0]] * len(bases_v) if val_v0 else bases_v
    return _ORIG_VERSIONS(q, bk, bv, versions, c_k, c_v, k_a, v_a, scale)


_ORIG_VERSIONS = lo.oracle_decode_unit_versions


def _q8_variant(x, rounding="even", divisor=127, qmax=127):
    x = np.asarray(x, np.float32)
    s = (np.max(np.abs(x), axis=1) / np.float32(divisor)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1)).astype(np.float32)
    t = x / safe[:, None]
    qf = np.sign(t) * np.floor(np.abs(t) + 0.5) if rounding == "away" else np.rint(t)
    q = np.clip(qf, -qmax, qmax)
    q[s == 0] = 0
    return q.astype(np.int8), s


def _gqa_modulo(q, bases_k, bases_v, codes_k, codes_v, anchors_k, anchors_v, scale=None):
    q = np.asarray(q, np.float64)
    batch, n_q, _ = q.shape
    n_kv = len(bases_k)
    scale = lo.default_scale() if scale is None else scale
    out = np.empty((batch, n_q, 128))
    for b in range(batch):
        for i in range(n_q):
            h = i % n_kv
            out[b, i] = lo.oracle_decode_unit(q[b, i:i + 1], bases_k[h], bases_v[h], codes_k[b][h],
                                              codes_v[b][h], anchors_k[b][h], anchors_v[b][h], scale)[0]
    return out


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    if name == "values_through_key_basis":
        # value accumulation reads the key codes instead of the value codes
        orig = lo.rank_space_values
        monkeypatch.setattr(lo, "oracle_decode_unit", _values_from_keys(orig))
        monkeypatch.setattr(oracle, "oracle_decode_unit", lo.oracle_decode_unit)
    elif name == "gqa_modulo_mapping":
        monkeypatch.setattr(lo, attr, _gqa_modulo)
        monkeypatch.setattr(oracle, attr, _gqa_modulo)
    else:
        monkeypatch.setattr(lo, attr, fn)
        if hasattr(oracle, attr):
            monkeypatch.setattr(oracle, attr, fn)
    assert _any_pin_fails(), f"mutant {name} survived every pin"


def _values_from_keys(_orig):
    def decode(q, u_k, u_v, c_k, c_v, k_a, v_a, scale, return_p=False):
        c = np.asarray(c_k).shape[0]
        qt = lo.project_query(q, u_k)
        s = np.concatenate([lo.code_scores(qt, c_k, scale), lo.anchor_scores(q, k_a, scale)], axis=1)
        e, tot = lo.softmax_weights(s)
        out = (lo.up_project(lo.rank_space_values(e[:, :c], c_k), u_k) + lo.anchor_values(e[:, c:], v_a)) / tot
        return (out, e / tot) if return_p else out
    return decode


def test_unmutated_oracle_passes_every_pin():
    assert not _any_pin_fails()
