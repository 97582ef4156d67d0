"""Seeded synthetic inputs for low-rank-compressed KV decode attention.

This package only *draws* inputs: rotations, decaying-spectrum keys and values,
calibration bases, queries and rank assignments.  It holds none of the method's
arithmetic (no projection into codes, no scores, no softmax), so both the CPU
oracle side and the GPU side of the tests can consume its output without sharing
any code of the method itself.
"""

from .workloads import (  # noqa: F401
    HEAD_DIM,
    WORKLOADS,
    Workload,
    basis,
    calibration_rows,
    group_basis,
    haar_orthogonal,
    layer_kv_device,
    queries,
    ranks,
    round_to_storage,
    rotation,
    spectrum,
    unit_kv,
    workload,
)
