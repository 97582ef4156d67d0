"""Online basis adaptation on the GPU (lrkv_oja_update) against the oracle's
Oja step (oracle.oja_update), on the same bf16 rows and the same bf16 basis.

The GPU works in float32 and stores the new basis in bf16; the oracle's float64
result rounded to bf16 must match within one bf16 step plus the float32 error
of the computation (an absolute 4e-6 for entries of unit-norm columns: it
matters only for entries so small that their bf16 step is finer), and bit for
bit almost everywhere (a float32 result next to a rounding boundary may round
the other way).
"""

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import D, announce
from rank_kv_cache_lrkv_amd import binding as B, layout

pytestmark = pytest.mark.gpu

W = synth.WORKLOADS


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16)


def bf16_ulp(x):
    _, e = np.frexp(np.abs(x))
    return np.ldexp(1.0, np.maximum(e, -125) - 8)


def random_basis(rng, r):
    q, _ = np.linalg.qr(rng.standard_normal((D, D)))
    return q[:, :r]


def read_basis(L, version, h, which):
    """(128, r) float64 basis of version `version`, head h, from the device buffer."""
    uk, uv = layout.bases_offsets(L.rank_k, L.rank_v)
    r = int((L.rank_k if which == 0 else L.rank_v)[h])
    off = version * layout.bases_elems(L.rank_k, L.rank_v) + int((uk if which == 0 else uv)[h])
    rows = L.bases[off:off + r * D].float().cpu().numpy().astype(np.float64).reshape(r, D)
    return rows.T


def make(rng, batch, n_kv, rk, rv, n_versions=2):
    L = B.Layer.allocate(dtype=B.LRKV_BF16, batch=batch, n_q_heads=n_kv, n_kv_heads=n_kv, window=4, cap=32,
                         rank_k=rk, rank_v=rv, n_versions=n_versions)
    u_k = [oracle.bf16_round(random_basis(rng, r)) for r in rk]
    u_v = [oracle.bf16_round(random_basis(rng, r)) for r in rv]
    flat = layout.pack_bases(u_k, u_v)
    L.bases[:flat.size] = bf16(flat).cuda()
    return L, u_k, u_v


def rows(rng, batch, n_kv, n, tau=16.0):
    sig = np.exp(-np.arange(D) / tau)
    out = np.empty((batch, n_kv, n, D), np.float32)
    for h in range(n_kv):
        rot = random_basis(rng, D)
        for b in range(batch):
            out[b, h] = (rng.standard_normal((n, D)) * sig) @ rot.T
    return oracle.bf16_round(out).astype(np.float32)


F32_ABS = 4e-6   # float32 error of one step on unit-norm columns


def check_basis(got, want64, label):
    want = oracle.bf16_round(want64)
    err = np.abs(got - want)
    worst = float(np.max(err / (bf16_ulp(want + 1e-30) + F32_ABS)))
    equal = float(np.mean(got == want))
    print(f"[parity] {label}: worst {worst:.2f} bf16 steps, bit-equal {equal:.4f}", flush=True)
    assert worst <= 1.0, (label, worst)
    assert equal >= 0.98, (label, equal)
    g = got.T @ got
    assert np.max(np.abs(g - np.eye(g.shape[0]))) < 0.05, label   # orthonormal up to bf16 storage


@pytest.mark.parametrize("which", [0, 1])
def test_oja_update_matches_oracle(which):
    rng = np.random.default_rng(40 + which)
    rk, rv = [16, 64, 128], [32, 16, 96]
    batch, n = 2, 300
    L, u_k, u_v = make(rng, batch, 3, rk, rv)
    x = rows(rng, batch, 3, n)
    xd = bf16(x).cuda()
    eta = 0.3
    announce(f"oja update which={which} ranks {rk}/{rv} batch {batch} n {n}")
    B.lrkv_oja_update(L, which, xd, n, eta, 0, 1)
    torch.cuda.synchronize()
    for h in range(3):
        u0 = (u_k if which == 0 else u_v)[h]
        want = oracle.oja_update(u0, x[:, h].reshape(-1, D).astype(np.float64), eta)
        check_basis(read_basis(L, 1, h, which), want, f"which{which}/h{h}")
        # version 0 is untouched, and so is the other matrix of version 1
        assert np.array_equal(read_basis(L, 0, h, which), u0)
        assert not read_basis(L, 1, h, 1 - which).any()


def test_oja_in_place_and_repeated_steps():
    """version_out == version_in gives the same bits as writing elsewhere; three
    chained in-place steps each match the oracle's step taken from the basis the
    device held before it (one bf16 rounding that lands the other way at one step
    is carried and grown by the next steps, so a chain is compared step by step,
    each at the single-step bar)."""
    rng = np.random.default_rng(43)
    rk, rv = [64, 32], [32, 32]
    L, u_k, _ = make(rng, 1, 2, rk, rv)
    L2, _, _ = make(np.random.default_rng(43), 1, 2, rk, rv)
    x = rows(rng, 1, 2, 200)
    xd = bf16(x).cuda()
    announce("oja in place vs out of place; three chained steps")
    B.lrkv_oja_update(L, 0, xd, 200, 0.5, 0, 1)
    B.lrkv_oja_update(L2, 0, xd, 200, 0.5, 0, 0)
    torch.cuda.synchronize()
    for h in range(2):
        assert np.array_equal(read_basis(L, 1, h, 0), read_basis(L2, 0, h, 0))
        want = oracle.oja_update(u_k[h], x[:, h].reshape(-1, D).astype(np.float64), 0.5)
        check_basis(read_basis(L2, 0, h, 0), want, f"chain step 1 h{h}")
    for step in (2, 3):
        before = [read_basis(L2, 0, h, 0) for h in range(2)]
        B.lrkv_oja_update(L2, 0, xd, 200, 0.5, 0, 0)
        torch.cuda.synchronize()
        for h in range(2):
            want = oracle.oja_update(before[h], x[:, h].reshape(-1, D).astype(np.float64), 0.5)
            check_basis(read_basis(L2, 0, h, 0), want, f"chain step {step} h{h}")


def test_oja_one_row_and_strided_input():
    """A single row (N = 1) read through a strided view (every other token)."""
    rng = np.random.default_rng(44)
    L, u_k, _ = make(rng, 1, 1, [32], [16])
    x = rows(rng, 1, 1, 8)
    xd = bf16(x).cuda()[:, :, ::2]
    announce("oja one row, strided")
    B.lrkv_oja_update(L, 0, xd, 1, 0.9, 0, 1)
    torch.cuda.synchronize()
    want = oracle.oja_update(u_k[0], x[0, 0, :1].astype(np.float64), 0.9)
    check_basis(read_basis(L, 1, 0, 0), want, "one_row")


def test_oja_full_prefill_llama_32k_sampled():
    """One step over the whole 32K-token prefill of the Llama-3.1-8B-shaped layer
    (4 rows x 32768 keys per KV head), sampled heads against the oracle."""
    w = W["llama31_8b_32k"]
    rk, rv = synth.ranks(w, 0)
    L = B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads, n_kv_heads=w.n_kv_heads,
                         window=w.window, cap=32, rank_k=rk, rank_v=rv, n_versions=2)
    u_k = [synth.basis(w, 0, h, "k", int(rk[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    u_v = [synth.basis(w, 0, h, "v", int(rv[h])).astype(np.float64) for h in range(w.n_kv_heads)]
    flat = layout.pack_bases(u_k, u_v)
    L.bases[:flat.size] = bf16(flat).cuda()
    K = torch.empty((w.batch, w.n_kv_heads, w.n_ctx, D), dtype=torch.bfloat16, device="cuda")
    for b in range(w.batch):
        for h in range(w.n_kv_heads):
            K[b, h] = bf16(synth.unit_kv(w, 0, h, b, "k")[:w.n_ctx]).cuda()
    announce(f"oja full prefill: {w.batch} x {w.n_ctx} keys per head")
    B.lrkv_oja_update(L, 0, K, w.n_ctx, 0.5, 0, 1)
    torch.cuda.synchronize()
    for h in (0, w.n_kv_heads - 1):
        x = np.concatenate([synth.unit_kv(w, 0, h, b, "k")[:w.n_ctx] for b in range(w.batch)]).astype(np.float64)
        want = oracle.oja_update(u_k[h], x, 0.5)
        check_basis(read_basis(L, 1, h, 0), want, f"full_prefill/h{h}")
