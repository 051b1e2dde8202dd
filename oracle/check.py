"""Parity criterion for C = A @ B (TEST INFRASTRUCTURE ONLY).

err = max_ij |C[i,j] - Cref[i,j]| / D[i,j],  D[i,j] = sum_k |A_ik| |B_kj|,
computed in fp64 from the oracle's Cref and D. Where D[i,j] == 0 every product
is zero, the exact result is 0, and C[i,j] must be exactly 0 (the entry then
contributes 0 to the maximum). Any non-finite value in C is a failure, since the
checked problems have finite inputs.
"""
from __future__ import annotations

import numpy as np

TOL = {"f32": 1e-5, "f16": 1e-4, "bf16": 1e-4}


def normalized_error(C, Cref, D) -> float:
    C = np.asarray(C, dtype=np.float64)
    if C.shape != Cref.shape:
        raise ValueError(f"shape mismatch {C.shape} vs {Cref.shape}")
    if C.size == 0:
        return 0.0
    if not np.all(np.isfinite(C)):
        return float("inf")
    diff = np.abs(C - Cref)
    zero = D == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(zero, 0.0, diff / np.where(zero, 1.0, D))
    return float(r.max())
