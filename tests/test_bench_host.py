"""Host-side checks of bench.py (no GPU): the one-GPU guard and the algorithmic
byte counts that the roofline's achieved bandwidth divides by, each written out
here from the per-unit figures (code rows, anchor rows, U_K, q) rather than taken
from bench.py's own arithmetic."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


# Llama-3.1-8B-shaped layer at 32K: batch 4, 8 KV heads, 32 query heads, window 128,
# rank_k 64, rank_v 32.  Code slots hold tokens 1 .. n - W - 1, anchors token 0 and
# the last W tokens.
B_, HKV, HQ, N, W, RK, RV = 4, 8, 32, 32768, 128, 64, 32
C = N - 1 - W            # 32,639 code rows per (row, KV head)
A = 1 + W                # 129 anchor rows per (row, KV head)
ANCHORS = B_ * HKV * A * 2 * 128 * 2          # keys and values, bf16
U_K = HKV * 128 * RK * 2
Q = B_ * HQ * 128 * 2


@pytest.mark.parametrize("label,kw,expected", [
    # bf16 codes: (r_k + r_v) bf16 values per code row
    ("bf16", {}, B_ * HKV * C * (RK + RV) * 2 + ANCHORS + U_K + Q),
    # int8 codes: r_k + r_v bytes plus a 4-byte scale for keys and for values
    ("int8", {"bits": 8}, B_ * HKV * C * ((RK + RV) + 8) + ANCHORS + U_K + Q),
    # 4-bit codes: half a byte per code plus the two scales
    ("int4", {"bits": 4}, B_ * HKV * C * ((RK + RV) // 2 + 8) + ANCHORS + U_K + Q),
    # two KV heads per code stream: half the code rows, the same anchors and U_K bytes
    ("hg2", {"hg": 2}, (B_ * HKV // 2) * C * (RK + RV) * 2 + ANCHORS + U_K + Q),
    # LowRAM, 4 residual rows (bf16, 128 wide, 4-byte slot) per 32-slot block, key codes only
    ("lowram4", {"resid": 4},
     B_ * HKV * (C * RK * 2 + ((C + 31) // 32) * 4 * (128 * 2 + 4)) + ANCHORS + U_K + Q),
    # codes under 3 basis versions: every version's U_K rows
    ("versions3", {"versions": 3}, B_ * HKV * C * (RK + RV) * 2 + ANCHORS + 3 * U_K + Q),
])
def test_partials_algorithmic_bytes(label, kw, expected):
    w = synth.WORKLOADS["llama31_8b_32k"]
    assert (w.batch, w.n_kv_heads, w.n_q_heads, w.n_ctx, w.window, w.rank_k, w.rank_v) == \
        (B_, HKV, HQ, N, W, RK, RV)
    got = bench.algorithmic_bytes(w, w.n_ctx, **kw)["partials"]
    assert got == expected, (label, got, expected)


def test_headline_bytes_value():
    # the figure quoted for the code-space kernel's roofline
    w = synth.WORKLOADS["llama31_8b_32k"]
    assert bench.algorithmic_bytes(w, w.n_ctx)["partials"] == 202_811_392
