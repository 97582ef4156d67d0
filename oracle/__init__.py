"""CPU oracle (float64 NumPy).  TEST INFRASTRUCTURE ONLY: imported by tests/,
``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg, never by the
library.  See lrkv_oracle.py for what it follows and what pins it."""

from .lrkv_oracle import (  # noqa: F401
    HEAD_DIM,
    anchor_positions,
    anchor_scores,
    anchor_values,
    bf16_round,
    code_positions,
    code_scores,
    compressed_unit_bytes,
    default_scale,
    dequantize_codes_q4,
    dequantize_codes_q8,
    full_kv_bytes,
    oracle_compress,
    oracle_decode_layer,
    oracle_decode_unit,
    project_query,
    quantize_codes_q4,
    quantize_codes_q8,
    rank_space_values,
    softmax_weights,
    up_project,
)
