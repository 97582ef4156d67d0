"""Workload table and seeded generators.

Keys and values are post-RoPE-like rows with a decaying singular spectrum:
each row is ``(z * sigma) @ R.T`` with ``z ~ N(0, I_128)``, ``sigma_i = exp(-i / tau)``
and ``R`` a Haar-random orthogonal matrix drawn once per (layer, KV head, role).
The per-head bases are the top-r right singular vectors of a separate 1024-row
calibration set drawn from the same distribution (the calibration-only SVD
projection of the "Half the Memory, None of the Answers Lost" blog, section 05:
keep the top-r directions of each head's statistics).

Everything is seeded through ``np.random.SeedSequence`` with a per-purpose key,
so any (layer, head, batch row) can be regenerated on its own.  Values in bf16
workloads are rounded to bf16 by torch's float->bfloat16 conversion, which is
round-to-nearest-even; the values are returned as float32 arrays holding exactly
bf16-representable numbers, so a float64 upcast is exact on both sides.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional, Tuple

import numpy as np

HEAD_DIM = 128

# role keys of the seed sequences
_ROLE = {
    "rot_k": 1,
    "rot_v": 2,
    "cal_k": 3,
    "cal_v": 4,
    "tok_k": 5,
    "tok_v": 6,
    "query": 7,
    "ranks": 8,
    "vmap": 9,
}


@dataclass(frozen=True)
class Workload:
    """One synthetic workload.  ``n_ctx`` counts cached tokens including the
    decode token; ``n_steps`` extra decode steps append one token each."""

    name: str
    wid: int                      # numeric id folded into every seed
    batch: int
    n_q_heads: int
    n_kv_heads: int
    n_ctx: int
    window: int
    dtype: str                    # "f32" or "bf16"
    rank_k: int = 64              # uniform ranks (ignored when mixed_ranks)
    rank_v: int = 32
    tau_k: float = 16.0
    tau_v: float = 16.0
    n_layers: int = 1
    n_steps: int = 0
    n_splits: Optional[int] = None
    mixed_ranks: bool = False
    rank_k_choices: Tuple[int, ...] = (32, 48, 64, 96)
    rank_v_choices: Tuple[int, ...] = (16, 32)
    v_from_k: float = 0.0         # values = a (keys @ Q) + sqrt(1 - a^2) (independent rows), Q orthogonal
    description: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_total(self) -> int:
        """Tokens generated per (layer, KV head, batch row): prefill plus appended steps."""
        return self.n_ctx + self.n_steps

    def scaled(self, **kw) -> "Workload":
        """Same recipe at another size (a parity case at reduced shape)."""
        d = {f: getattr(self, f) for f in self.__dataclass_fields__}
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    w.name: w
    for w in [
        Workload(
            name="tiny_f32", wid=1, batch=1, n_q_heads=1, n_kv_heads=1, n_ctx=256,
            window=16, dtype="f32", rank_k=64, rank_v=32,
            description="single head, fp32 storage, anchors = first token + last 16",
        ),
        Workload(
            name="qwen3_1p7b_4k", wid=2, batch=8, n_q_heads=16, n_kv_heads=8, n_ctx=4096,
            window=64, dtype="bf16", rank_k=64, rank_v=32,
            description="Qwen3-1.7B-shaped layer, GQA group 2, 4K context",
        ),
        Workload(
            name="llama31_8b_32k", wid=3, batch=4, n_q_heads=32, n_kv_heads=8, n_ctx=32768,
            window=128, dtype="bf16", rank_k=64, rank_v=32, n_splits=32,
            description="Llama-3.1-8B-shaped layer, GQA group 4, 32K context, 32 splits",
        ),
        Workload(
            name="llama31_8b_hc_8k", wid=4, batch=64, n_q_heads=32, n_kv_heads=8, n_ctx=8192,
            window=32, dtype="bf16", rank_k=32, rank_v=16, tau_k=32.0,
            description="high-compression regime, batch 64, 8K context, slower key decay",
        ),
        Workload(
            name="llama31_8b_32layer", wid=5, batch=4, n_q_heads=32, n_kv_heads=8,
            n_ctx=32768, window=128, dtype="bf16", n_layers=32, n_steps=16,
            mixed_ranks=True,
            description="32-layer prefill compression, then 16 decode steps, mixed ranks",
        ),
    ]
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


def _rng(w: Workload, role: str, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([w.wid, _ROLE[role], *key]))


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round to the storage type; returns float32 holding the stored values."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        import torch

        t = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float32)
        return t.numpy()
    raise ValueError(dtype)


def spectrum(tau: float) -> np.ndarray:
    return np.exp(-np.arange(HEAD_DIM, dtype=np.float64) / tau)


def haar_orthogonal(rng: np.random.Generator, d: int = HEAD_DIM) -> np.ndarray:
    """Haar-distributed orthogonal matrix: QR of a Gaussian matrix with the
    signs of R's diagonal folded into Q (Mezzadri, 2007)."""
    a = rng.standard_normal((d, d))
    qm, rm = np.linalg.qr(a)
    return qm * np.sign(np.diag(rm))[None, :]


def ranks(w: Workload, layer: int) -> Tuple[np.ndarray, np.ndarray]:
    """Per-KV-head (r_k, r_v) for one layer."""
    if not w.mixed_ranks:
        return (np.full(w.n_kv_heads, w.rank_k, dtype=np.int32),
                np.full(w.n_kv_heads, w.rank_v, dtype=np.int32))
    g = _rng(w, "ranks", layer)
    rk = g.choice(np.asarray(w.rank_k_choices), size=w.n_kv_heads)
    rv = g.choice(np.asarray(w.rank_v_choices), size=w.n_kv_heads)
    return rk.astype(np.int32), rv.astype(np.int32)


def rotation(w: Workload, layer: int, head: int, which: str) -> np.ndarray:
    return haar_orthogonal(_rng(w, "rot_" + which, layer, head))


def _tau(w: Workload, which: str) -> float:
    return w.tau_k if which == "k" else w.tau_v


def calibration_rows(w: Workload, layer: int, head: int, which: str, n_cal: int = 1024) -> np.ndarray:
    """The separate calibration set (float64, unrounded)."""
    z = _rng(w, "cal_" + which, layer, head).standard_normal((n_cal, HEAD_DIM))
    return (z * spectrum(_tau(w, which))[None, :]) @ rotation(w, layer, head, which).T


def basis(w: Workload, layer: int, head: int, which: str, rank: int) -> np.ndarray:
    """U = top-``rank`` right singular vectors of the calibration rows, as a
    (128, rank) matrix with orthonormal columns, rounded to storage."""
    x = calibration_rows(w, layer, head, which)
    _, _, vt = np.linalg.svd(x, full_matrices=False)
    return round_to_storage(vt[:rank].T, w.dtype)


def group_basis(w: Workload, layer: int, group: int, head_group: int, which: str, rank: int) -> np.ndarray:
    """Basis of a group of ``head_group`` consecutive KV heads (group-head
    latents): the top-``rank`` right singular vectors of the group's calibration
    rows joined feature-wise (head by head), a (128 * head_group, rank) matrix
    with orthonormal columns, rounded to storage."""
    heads = range(group * head_group, (group + 1) * head_group)
    x = np.concatenate([calibration_rows(w, layer, h, which) for h in heads], axis=1)
    _, _, vt = np.linalg.svd(x, full_matrices=False)
    return round_to_storage(vt[:rank].T, w.dtype)


def _raw_rows(w: Workload, layer: int, head: int, b: int, which: str) -> np.ndarray:
    z = _rng(w, "tok_" + which, layer, head, b).standard_normal((w.n_total, HEAD_DIM))
    return (z * spectrum(_tau(w, which))[None, :]) @ rotation(w, layer, head, which).T


def unit_kv(w: Workload, layer: int, head: int, b: int, which: str) -> np.ndarray:
    """All ``n_total`` rows of keys (``which='k'``) or values for one
    (layer, KV head, batch row), rounded to storage: shape (n_total, 128).
    With ``v_from_k`` = a > 0 the values are partly a fixed orthogonal map of the
    keys (the structure LowRAM's value amortisation relies on)."""
    x = _raw_rows(w, layer, head, b, which)
    if which == "v" and w.v_from_k > 0:
        a = float(w.v_from_k)
        q = haar_orthogonal(_rng(w, "vmap", layer, head))
        x = a * (_raw_rows(w, layer, head, b, "k") @ q) + np.sqrt(max(0.0, 1.0 - a * a)) * x
    return round_to_storage(x, w.dtype)


def queries(w: Workload, layer: int, step: int, b: int, scale: float = 1.0) -> np.ndarray:
    """Decode queries of all query heads of one batch row: (n_q_heads, 128).
    ``scale`` > 1 sharpens the attention (a peaky-softmax stress case)."""
    q = _rng(w, "query", layer, step, b).standard_normal((w.n_q_heads, HEAD_DIM)) * scale
    return round_to_storage(q, w.dtype)


def layer_kv_device(w: Workload, layer: int, which: str, device="cuda"):
    """Keys or values of every (batch row, KV head) of one layer drawn on the GPU:
    a torch bfloat16 tensor [batch][n_kv_heads][n_total][128] of rows
    (z * sigma) R^T with the same spectrum and the same Haar rotation per
    (layer, KV head) as ``unit_kv``, but latents z from torch's device generator
    (seeded per (layer, KV head, role)), multiplied in float32.  Same
    distribution as ``unit_kv``, other random draws: for inputs too large to make
    on the host in reasonable time (the 32-layer cache), where no oracle reads
    them."""
    import torch

    assert w.v_from_k == 0.0, "device generation has no key-to-value map"
    out = torch.empty((w.batch, w.n_kv_heads, w.n_total, HEAD_DIM), dtype=torch.bfloat16, device=device)
    sig = torch.from_numpy(spectrum(_tau(w, which)).astype(np.float32)).to(device)
    gen = torch.Generator(device=device)
    for h in range(w.n_kv_heads):
        seed = int(np.random.SeedSequence([w.wid, _ROLE["tok_" + which], layer, h, 1 << 20])
                   .generate_state(1, np.uint64)[0] >> np.uint64(1))
        gen.manual_seed(seed)
        rt = torch.from_numpy(rotation(w, layer, h, which).T.astype(np.float32)).to(device)
        z = torch.randn((w.batch, w.n_total, HEAD_DIM), generator=gen, device=device, dtype=torch.float32)
        out[:, h] = ((z * sig) @ rt).to(torch.bfloat16)
        del z
    return out
