"""Host-side helpers for the buffer layouts of include/lrkv.h (NumPy, no GPU).

Used to size buffers and to move codes between the logical (tokens, rank)
view and the blocked order the kernels read.
"""

from __future__ import annotations

from typing import Sequence

import numpy as np

HEAD_DIM = 128
BLOCK = 32


def round_cap(n: int) -> int:
    """Smallest valid capacity (a multiple of 32 slots) holding n codes."""
    n = max(0, int(n))
    return (n + BLOCK - 1) // BLOCK * BLOCK


def bases_elems(rank_k: Sequence[int], rank_v: Sequence[int], head_group: int = 1) -> int:
    """Elements of one version of the bases: per head (or head group of
    ``head_group`` KV heads) U_K^T and U_V^T with rows of 128 * head_group."""
    return HEAD_DIM * int(head_group) * int(np.sum(rank_k) + np.sum(rank_v))


def bases_offsets(rank_k: Sequence[int], rank_v: Sequence[int], head_group: int = 1):
    """Element offsets of U_K(h) and U_V(h) (h a head, or a head group) in the
    bases buffer."""
    row = HEAD_DIM * int(head_group)
    uk, uv, off = [], [], 0
    for rk, rv in zip(rank_k, rank_v):
        uk.append(off)
        uv.append(off + row * int(rk))
        off += row * (int(rk) + int(rv))
    return np.array(uk), np.array(uv)


def pack_bases(u_k: Sequence[np.ndarray], u_v: Sequence[np.ndarray]) -> np.ndarray:
    """Flat bases buffer from per-head (128, r) matrices (per head group:
    (128 * head_group, r)): head by head, U_K^T then U_V^T, each basis direction
    as its rows' contiguous elements."""
    parts = []
    for uk, uv in zip(u_k, u_v):
        parts += [np.asarray(uk).T.ravel(), np.asarray(uv).T.ravel()]
    return np.concatenate(parts) if parts else np.zeros(0)


def codes_elems(ranks: Sequence[int], batch: int, cap: int) -> int:
    return int(batch) * int(cap) * int(np.sum(ranks))


def code_offsets(ranks: Sequence[int], batch: int, cap: int) -> np.ndarray:
    """Element offset of head h's [batch][cap][r] region in a codes buffer."""
    r = np.asarray(ranks, np.int64)
    return np.concatenate([[0], np.cumsum(int(batch) * int(cap) * r)[:-1]]).astype(np.int64)


def scales_elems(n_kv_heads: int, batch: int, cap: int) -> int:
    """Elements of one quantised-code scales buffer: float32 [heads][batch][cap]
    (heads = KV heads, or latent groups with head groups)."""
    return int(n_kv_heads) * int(batch) * int(cap)


def scale_offset(h: int, b: int, cap: int, batch: int) -> int:
    """Element offset of slot 0 of (KV head or latent group h, batch row b) in a
    scales buffer."""
    return (int(h) * int(batch) + int(b)) * int(cap)


def predictor_elems(rank_k: Sequence[int], batch: int) -> int:
    """Elements of a LowRAM predictor buffer: M(b, h), rank_k[h] rows of 128."""
    return HEAD_DIM * int(batch) * int(np.sum(rank_k))


def predictor_offset(rank_k: Sequence[int], batch: int, h: int, b: int) -> int:
    """Element offset of M(b, h)'s first row."""
    r = np.asarray(rank_k, np.int64)
    return int(HEAD_DIM * (int(batch) * int(np.sum(r[:h])) + int(b) * int(r[h])))


def resid_entries(n_kv_heads: int, batch: int, cap: int, r: int) -> int:
    """LowRAM residual entries: R per 32-slot block of every (KV head, row)."""
    return int(n_kv_heads) * int(batch) * (int(cap) // BLOCK) * int(r)


def resid_entry(h: int, b: int, blk: int, i: int, batch: int, cap: int, r: int) -> int:
    """Index of entry i of block blk of (KV head h, row b)."""
    return ((int(h) * int(batch) + int(b)) * (int(cap) // BLOCK) + int(blk)) * int(r) + int(i)


def block_positions(r: int, which: str) -> np.ndarray:
    """In-block element position of (slot t in 0..31, column c in 0..r-1)."""
    t = np.arange(BLOCK)[:, None]
    c = np.arange(r)[None, :]
    if which == "k":
        return ((t // 16) * (r // 8) + c // 8) * 128 + (t % 16) * 8 + c % 8
    if which == "v":
        return ((t % 16) // 4 * r + c) * 8 + 4 * (t // 16) + t % 4
    raise ValueError(which)


def slot_positions(n: int, r: int, which: str) -> np.ndarray:
    """Element position of (slot j in 0..n-1, column c) inside one (row, head) region."""
    j = np.arange(n)
    return (j // BLOCK)[:, None] * (BLOCK * r) + block_positions(r, which)[j % BLOCK]


def pack_codes(codes: np.ndarray, cap: int, which: str) -> np.ndarray:
    """(n, r) logical codes of slots 0..n-1 -> flat (cap * r) blocked region."""
    n, r = codes.shape
    assert n <= cap and cap % BLOCK == 0
    out = np.zeros(cap * r, dtype=codes.dtype)
    out[slot_positions(n, r, which)] = codes
    return out


def pack_nibbles(values: np.ndarray) -> np.ndarray:
    """Flat element array of 4-bit values in [-8, 7] -> bytes, two per byte, even
    elements in the low four bits (the 4-bit code layout of lrkv.h)."""
    v = np.asarray(values).astype(np.int16) & 0xF
    if v.size % 2:
        v = np.concatenate([v, np.zeros(1, v.dtype)])
    return (v[0::2] | (v[1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Bytes -> flat element array of signed 4-bit values (int8)."""
    b = np.asarray(packed, np.uint8).astype(np.int16)
    v = np.empty(b.size * 2, np.int16)
    v[0::2] = b & 0xF
    v[1::2] = b >> 4
    return np.where(v >= 8, v - 16, v).astype(np.int8)


def unpack_codes(region: np.ndarray, n: int, r: int, which: str) -> np.ndarray:
    """Flat blocked region -> (n, r) logical codes of slots 0..n-1."""
    return np.asarray(region)[slot_positions(n, r, which)]


def anchor_slot(p: int, window: int) -> int:
    return 0 if p == 0 else 1 + (p - 1) % window
