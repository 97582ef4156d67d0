"""The allocation-free decode entry point (lrkv_decode_attn_noalloc) through the
C ABI: its output against lrkv_decode_attn's (same kernels, same splits, so
bitwise the same; the decode bar is checked too) on two calls in a row, the
second on a smaller input, and the host-side rejection of a call whose split
records exceed the library's array."""

import numpy as np
import pytest
import torch

import oracle
import synth
from cases import D, announce, check_decode, dev, gpu_layer, host_case
from rank_kv_cache_lrkv_amd import binding as B

pytestmark = pytest.mark.gpu


def run_both(hc, S):
    L = gpu_layer(hc)
    w = hc.w
    q = dev(hc.q, w.dtype)
    ref = torch.empty((w.batch, w.n_q_heads, D), dtype=torch.float32, device="cuda")
    got = torch.full_like(ref, float("nan"))
    B.lrkv_decode_attn(L, hc.n, q, ref, oracle.default_scale(), S, B.workspace(L, S))
    B.lrkv_decode_attn_noalloc(L, hc.n, q, got, oracle.default_scale(), S)
    torch.cuda.synchronize()
    return got.cpu().numpy().astype(np.float64), ref.cpu().numpy().astype(np.float64)


def test_noalloc_matches_decode_attn_twice():
    big = synth.WORKLOADS["llama31_8b_32k"].scaled(batch=2, n_ctx=3000)
    small = synth.WORKLOADS["qwen3_1p7b_4k"].scaled(batch=1, n_q_heads=4, n_kv_heads=2, n_ctx=300)
    for label, w, S in (("first, larger", big, 32), ("second, smaller", small, 0)):
        hc = host_case(w)
        S = S or B.lrkv_decode_auto_splits(gpu_layer(hc, with_codes=False), hc.n)
        announce(f"noalloc decode {label}: batch {w.batch} n {w.n_ctx} S {S}")
        got, ref = run_both(hc, S)
        assert np.array_equal(got, ref), label
        check_decode(got, hc.expected(), w.dtype, f"noalloc_{label}")


def test_noalloc_rejects_records_past_its_array():
    # 64 rows x 32 query heads x 1024 splits x (4 + 32 + 128) floats > 16 MiB
    w = synth.WORKLOADS["llama31_8b_hc_8k"].scaled(n_ctx=100)
    hc_layer = B.Layer.allocate(dtype=B.LRKV_BF16, batch=w.batch, n_q_heads=w.n_q_heads,
                                n_kv_heads=w.n_kv_heads, window=w.window, cap=96,
                                rank_k=[32] * 8, rank_v=[32] * 8)
    assert B.lrkv_decode_workspace_size(hc_layer, 1024) > B.NOALLOC_CAPACITY
    q = torch.zeros((w.batch, w.n_q_heads, D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((w.batch, w.n_q_heads, D), dtype=torch.float32, device="cuda")
    with pytest.raises(B.LrkvError) as e:
        B.lrkv_decode_attn_noalloc(hc_layer, 100, q, out, oracle.default_scale(), 1024)
    assert e.value.status == 7
    assert torch.all(out == 0)
