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


# Rounding unit of a stored output type (half an ulp relative, round to nearest even).
OUT_UNIT = {"f32": 0.0, "f16": 2.0 ** -11, "bf16": 2.0 ** -8}
# Smallest positive subnormal spacing of the output type (absolute floor of its rounding).
OUT_TINY = {"f32": 0.0, "f16": 2.0 ** -25, "bf16": 2.0 ** -134}


def epilogue_error(C, ref, Dp, in_dtype: str, out_dtype: str) -> float:
    """Largest ratio |C - ref| / bound over all entries; <= 1 passes.

    bound = 1.2 TOL[in] Dp + 1e-6 Dp + OUT_UNIT[out] |ref| + OUT_TINY[out]:
    the product's normalized tolerance scaled through alpha, the fp32 rounding of
    the epilogue's own operations (a few units of 2^-24 of Dp), the activation's
    Lipschitz constant (1 for ReLU, under 1.13 for GELU) and its fp32 evaluation,
    and the rounding of the stored value to the output type. Non-finite C fails.
    """
    C = np.asarray(C, dtype=np.float64)
    if C.shape != ref.shape:
        raise ValueError(f"shape mismatch {C.shape} vs {ref.shape}")
    if C.size == 0:
        return 0.0
    if not np.all(np.isfinite(C)):
        return float("inf")
    bound = (1.2 * TOL[in_dtype] + 1e-6) * Dp + OUT_UNIT[out_dtype] * np.abs(ref) + OUT_TINY[out_dtype]
    diff = np.abs(C - ref)
    zero = bound == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(zero, 0.0, diff / np.where(zero, 1.0, bound))
    return float(r.max())
