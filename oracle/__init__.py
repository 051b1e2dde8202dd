"""CPU oracle for the dense matrix product C = A @ B (TEST INFRASTRUCTURE ONLY).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never imports, links or
calls it, and it imports nothing from the GPU library: the two share only the
seeded input module ``gemm_inputs``.

``oracle_gemm.c`` holds the arithmetic: a plain triple loop in fp64 over
exactly decoded inputs (the definition of the product the chapter "Shared
memory and tensor cores" tiles in sections 13.1-13.3), plus the error
denominator sum_k |A_ik| |B_kj|. ``check.py`` holds the normalized error
max_ij |C - Cref| / D used as the parity criterion.

Parity status: every function here is pinned by tests that do not reuse its
code (exact Fraction sums, identity/permutation/rank-1 closed forms, integer
exactness, a float64 library product, and the chapter's printed fp16 precision
figures in section 13.8).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle_gemm.c")
_LIB = os.path.join(_HERE, "liboracle_gemm.so")
_DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2}
_lib = None


def compile_source(src: str, out: str) -> str:
    """gcc -O3 with OpenMP; no fast-math and no FMA contraction, so each sum rounds as written."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
           "-fno-fast-math", "-march=x86-64-v2", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle_gemm.c into liboracle_gemm.so next to it."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    return compile_source(_SRC, _LIB)


def open_library(path: str):
    """Open a compiled oracle library at `path` and declare its signatures."""
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_gemm.argtypes = [ctypes.c_int, ctypes.c_int, i64, i64, i64, vp, i64, vp, i64,
                                ctypes.c_int, vp, i64, vp, vp, ctypes.c_int]
    lib.oracle_gemm.restype = ctypes.c_int
    lib.oracle_decode16.argtypes = [ctypes.c_uint16, ctypes.c_int]
    lib.oracle_decode16.restype = ctypes.c_double
    lib.oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = open_library(_LIB)
    return _lib


def _ptr(a):
    return None if a is None or a.size == 0 else a.ctypes.data_as(ctypes.c_void_p)


def gemm_ref(ops, rows=None, want_d: bool = True, nthreads: int = 0, op_a: str = "N", lda=None, lib=None):
    """Cref (fp64) and D (fp64, or None) for an ``gemm_inputs.Operands`` problem.

    ``rows`` selects output rows (default: all M). Returns arrays of shape
    (len(rows), N).
    """
    lib = lib or _load()
    M, N, K = ops.M, ops.N, ops.K
    if rows is None:
        nrows = M
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    C = np.zeros((nrows, N), dtype=np.float64)
    D = np.zeros((nrows, N), dtype=np.float64) if want_d else None
    A = np.ascontiguousarray(ops.A)
    B = np.ascontiguousarray(ops.B)
    rc = lib.oracle_gemm(0 if op_a == "N" else 1, 0 if ops.op_b == "N" else 1, M, N, K,
                         _ptr(A), ops.lda if lda is None else lda, _ptr(B), ops.ldb,
                         _DTYPE_CODE[ops.dtype], _ptr(rows_arr), nrows, _ptr(C), _ptr(D), nthreads)
    if rc != 0:
        raise ValueError("oracle_gemm rejected its arguments")
    return C, D


def decode16(bits: int, dtype: str) -> float:
    """The oracle's own decode of one fp16/bf16 bit pattern."""
    return _load().oracle_decode16(int(bits), _DTYPE_CODE[dtype])


def max_threads() -> int:
    return _load().oracle_max_threads()


def timed_gemm_ref(ops, rows=None, nthreads: int = 0):
    """Run the Cref computation only (no D) and return (Cref, seconds)."""
    t0 = time.perf_counter()
    C, _ = gemm_ref(ops, rows=rows, want_d=False, nthreads=nthreads)
    return C, time.perf_counter() - t0
