"""Oracle of the fused epilogue (TEST INFRASTRUCTURE ONLY).

"Shared memory and tensor cores", section 13.10, lists epilogue fusion among what
production GEMM kernels add: a bias, an activation, a residual add or a type
cast applied to the accumulator before the store. The pages fix no order of
these steps; the reading used here (and by the library) is the BLAS-style one:

    C = act(alpha * (A @ B) + beta * R + bias[col])

computed here in fp64 from the oracle's exact product (``gemm_ref``), R decoded
exactly from its stored type. GELU is its tanh form (Hendrycks and Gimpel),
written as defined: x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3))).

Only tests, ``__graft_entry__.smoke()`` and bench.py's CPU baseline may use this
module; it shares nothing with the GPU library.
"""
from __future__ import annotations

import math

import numpy as np

ACTIVATIONS = ("none", "relu", "gelu_tanh")


def gelu_tanh(x):
    """GELU, tanh form, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


def epilogue_ref(Cref, D, alpha=1.0, beta=0.0, R=None, bias=None, act="none"):
    """(reference C, error scale Dp) for C = act(alpha * Cref + beta * R + bias).

    Cref, D: the oracle's exact product and its denominator sum_k |A_ik||B_kj| (fp64,
    M x N). R: M x N values (fp64) or None. bias: N values or None. Dp bounds the
    magnitude the fp32 arithmetic works on: |alpha| D + |beta| |R| + |bias|.
    """
    if act not in ACTIVATIONS:
        raise ValueError(f"unknown activation {act!r}")
    x = float(alpha) * np.asarray(Cref, dtype=np.float64)
    Dp = abs(float(alpha)) * np.asarray(D, dtype=np.float64)
    if beta != 0.0:
        R = np.asarray(R, dtype=np.float64)
        x = x + float(beta) * R
        Dp = Dp + abs(float(beta)) * np.abs(R)
    if bias is not None:
        b = np.asarray(bias, dtype=np.float64)[None, :]
        x = x + b
        Dp = Dp + np.abs(b)
    if act == "relu":
        x = np.maximum(x, 0.0)
    elif act == "gelu_tanh":
        x = gelu_tanh(x)
    return x, Dp
