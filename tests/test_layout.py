"""Host-side layout helpers against the layout stated in include/lrkv.h (no GPU)."""

import numpy as np

from rank_kv_cache_lrkv_amd import layout


def test_block_positions_are_a_permutation():
    for r in [16, 32, 48, 64, 96, 128]:
        for which in "kv":
            p = layout.block_positions(r, which)
            assert sorted(p.ravel().tolist()) == list(range(32 * r))


def test_key_blocks_group_eight_columns_of_one_token():
    r = 64
    p = layout.block_positions(r, "k")
    for t in range(32):
        for c0 in range(0, r, 8):
            run = p[t, c0:c0 + 8]
            assert np.array_equal(run, np.arange(run[0], run[0] + 8))
    # the 16 tokens of a half block follow each other within one 8-column group
    assert p[1, 0] - p[0, 0] == 8 and p[16, 0] == 16 * r


def test_value_blocks_group_eight_tokens_of_one_column():
    r = 32
    p = layout.block_positions(r, "v")
    for c in range(r):
        for q in range(4):
            toks = [16 * (j // 4) + 4 * q + j % 4 for j in range(8)]
            assert np.array_equal(p[toks, c], np.arange(p[toks[0], c], p[toks[0], c] + 8))


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(0)
    for r in [16, 48, 128]:
        for n, cap in [(0, 0), (1, 32), (31, 32), (70, 96)]:
            for which in "kv":
                codes = rng.standard_normal((n, r)).astype(np.float32)
                flat = layout.pack_codes(codes, cap, which)
                assert flat.shape == (cap * r,)
                assert np.array_equal(layout.unpack_codes(flat, n, r, which), codes)


def test_offsets():
    rk, rv = [64, 32, 96], [16, 32, 16]
    uk, uv = layout.bases_offsets(rk, rv)
    assert uk.tolist() == [0, 128 * 80, 128 * 144] and uv.tolist() == [128 * 64, 128 * 112, 128 * 240]
    assert layout.bases_elems(rk, rv) == 128 * 256
    assert layout.code_offsets(rk, 2, 64).tolist() == [0, 2 * 64 * 64, 2 * 64 * 96]
    assert layout.round_cap(0) == 0 and layout.round_cap(1) == 32 and layout.round_cap(64) == 64
    assert [layout.anchor_slot(p, 4) for p in range(9)] == [0, 1, 2, 3, 4, 1, 2, 3, 4]


def test_pack_bases_rows_are_basis_directions():
    rng = np.random.default_rng(1)
    uk = [rng.standard_normal((128, 32)), rng.standard_normal((128, 16))]
    uv = [rng.standard_normal((128, 16)), rng.standard_normal((128, 48))]
    flat = layout.pack_bases(uk, uv)
    assert flat.shape == (layout.bases_elems([32, 16], [16, 48]),)
    ok, ov = layout.bases_offsets([32, 16], [16, 48])
    for h in range(2):
        for c in range(uk[h].shape[1]):
            assert np.array_equal(flat[ok[h] + 128 * c: ok[h] + 128 * (c + 1)], uk[h][:, c])
        for c in range(uv[h].shape[1]):
            assert np.array_equal(flat[ov[h] + 128 * c: ov[h] + 128 * (c + 1)], uv[h][:, c])


def test_nibble_packing_round_trip_and_order():
    rng = np.random.default_rng(5)
    v = rng.integers(-8, 8, 1001).astype(np.int8)
    p = layout.pack_nibbles(v)
    assert p.dtype == np.uint8 and p.size == 501
    assert np.array_equal(layout.unpack_nibbles(p)[:1001], v)
    # element 0 in the low four bits, element 1 in the high four bits, two's complement
    assert layout.pack_nibbles(np.array([-1, 2], np.int8)).tolist() == [0x2F]
    assert layout.pack_nibbles(np.array([7, -8], np.int8)).tolist() == [0x87]
