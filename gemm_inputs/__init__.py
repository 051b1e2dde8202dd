"""Seeded synthetic operands for the dense GEMM C = A @ B.

This module only draws and stores numbers; it performs no part of the matrix
product. Both the CPU oracle (through the tests) and the GPU library consume
exactly the arrays it returns, so the two sides always see the same rounded
input values.

Conventions
-----------
* Generator: ``numpy.random.default_rng(seed)``, the generator the
  "Shared memory and tensor cores" chapter uses for its fp16 precision model
  (section 13.8). A is drawn first, then B, from the same generator.
* "uniform": ``rng.uniform(-1, 1)`` in float64, stored as float32; for fp16 the
  float32 values are rounded to nearest-even with ``astype(np.float16)`` (the
  chapter's own rounding step in 13.8); for bf16 they are rounded to
  nearest-even bfloat16.
* "normal": ``rng.standard_normal`` in float64, stored as float32, then rounded
  the same way.
* Storage: every operand is a flat array in its storage order. A is row-major
  with ``lda >= K``. B is either row-major ``K x N`` (op 'N', ``ldb >= N``) or
  column-major, i.e. a row-major ``N x K`` array (op 'T', ``ldb >= K``). Values
  are drawn in storage order over the logical rows and columns only; padding
  columns (``ld`` beyond the logical width) are filled with a NaN pattern so a
  kernel that reads them produces NaN.
* fp16 and bf16 operands are returned as ``uint16`` bit patterns; fp32 as
  ``float32``.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DTYPES = ("f32", "f16", "bf16")
ELEM_SIZE = {"f32": 4, "f16": 2, "bf16": 2}

# quiet-NaN patterns used to poison padding columns
_NAN_BITS = {"f32": np.uint32(0x7FC00000), "f16": np.uint16(0x7E00), "bf16": np.uint16(0x7FC0)}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the 16-bit patterns.

    NaN inputs map to a quiet NaN; infinities and overflow to infinity follow
    from the integer rounding carry.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded = rounded.copy()
        rounded[nan] = 0x7FC0
    return rounded


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (nearest-even) and return the bit patterns."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_storage(x32: np.ndarray, dtype: str) -> np.ndarray:
    """float32 values -> the storage array of `dtype` (float32, or uint16 bit patterns)."""
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "f16":
        return f32_to_f16_bits(x32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _draw(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "uniform":
        return rng.uniform(-1.0, 1.0, shape).astype(np.float32)
    if dist == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    raise ValueError(f"unknown distribution {dist!r}")


def _padded(vals: np.ndarray, ld: int, dtype: str) -> np.ndarray:
    """Place a (rows, cols) storage array into rows of length `ld`, padding with NaN patterns."""
    rows, cols = vals.shape
    if ld < cols:
        raise ValueError(f"leading dimension {ld} < row length {cols}")
    if ld == cols:
        return np.ascontiguousarray(vals).reshape(-1)
    out = np.empty((rows, ld), dtype=vals.dtype)
    if dtype == "f32":
        out.view(np.uint32)[:] = _NAN_BITS["f32"]
    else:
        out[:] = _NAN_BITS[dtype]
    out[:, :cols] = vals
    return out.reshape(-1)


@dataclass
class Operands:
    """Storage of one GEMM problem. `A` and `B` are flat arrays in storage order."""

    M: int
    N: int
    K: int
    dtype: str
    op_b: str
    lda: int
    ldb: int
    A: np.ndarray
    B: np.ndarray

    @property
    def elem_size(self) -> int:
        return ELEM_SIZE[self.dtype]


def make_operands(M: int, N: int, K: int, dtype: str = "f32", dist: str = "uniform", seed: int = 0,
                  op_b: str = "N", lda: int | None = None, ldb: int | None = None) -> Operands:
    """Draw A (M x K) then B (K x N, stored per `op_b`) from ``default_rng(seed)``."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    if op_b not in ("N", "T"):
        raise ValueError(f"op_b must be 'N' or 'T', got {op_b!r}")
    lda = max(1, K) if lda is None else lda
    if ldb is None:
        ldb = max(1, N) if op_b == "N" else max(1, K)
    rng = np.random.default_rng(seed)
    a32 = _draw(rng, dist, (M, K))
    b_shape = (K, N) if op_b == "N" else (N, K)
    b32 = _draw(rng, dist, b_shape)
    A = _padded(to_storage(a32, dtype).reshape(M, K), lda, dtype) if M * K else np.zeros(M * lda, _np_storage(dtype))
    B = _padded(to_storage(b32, dtype).reshape(b_shape), ldb, dtype) if K * N else np.zeros(b_shape[0] * ldb, _np_storage(dtype))
    return Operands(M, N, K, dtype, op_b, lda, ldb, A, B)


def from_values(a: np.ndarray, b: np.ndarray, dtype: str = "f32", op_b: str = "N",
                lda: int | None = None, ldb: int | None = None) -> Operands:
    """Wrap given logical matrices a (M x K) and b (K x N) as storage arrays.

    Values must already be representable in `dtype` if an exact problem is wanted
    (small integers are exact in all three dtypes).
    """
    a = np.asarray(a, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    M, K = a.shape
    K2, N = b.shape
    if K2 != K:
        raise ValueError("inner dimensions differ")
    lda = max(1, K) if lda is None else lda
    if ldb is None:
        ldb = max(1, N) if op_b == "N" else max(1, K)
    bs = b if op_b == "N" else np.ascontiguousarray(b.T)
    A = _padded(to_storage(a, dtype).reshape(M, K), lda, dtype) if M * K else np.zeros(M * lda, _np_storage(dtype))
    B = _padded(to_storage(bs, dtype).reshape(bs.shape), ldb, dtype) if K * N else np.zeros(bs.shape[0] * ldb, _np_storage(dtype))
    return Operands(M, N, K, dtype, op_b, lda, ldb, A, B)


def _np_storage(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


# The five benchmark problems: the dense GEMM workloads whose shapes, dtypes and
# value distributions the pages measure or discuss (4096^3 traffic model, the
# 1024^3 CPU benchmark shape, fp16-in/fp32-acc matrix-core GEMM) plus a ragged
# bf16 case with column-major B.
CONFIGS = {
    "c1_f32_256": dict(M=256, N=256, K=256, dtype="f32", dist="uniform", op_b="N"),
    "c2_f32_1024": dict(M=1024, N=1024, K=1024, dtype="f32", dist="uniform", op_b="N"),
    "c3_f32_4096": dict(M=4096, N=4096, K=4096, dtype="f32", dist="uniform", op_b="N"),
    "c4_f16_4096": dict(M=4096, N=4096, K=4096, dtype="f16", dist="uniform", op_b="N"),
    "c5_bf16_ragged": dict(M=3001, N=5003, K=1037, dtype="bf16", dist="normal", op_b="T"),
}

# Further workloads for the rows beyond the five problems: a long-K product with
# few output tiles (the case split K is for).
EXTRA_CONFIGS = {
    "k1_f32_long_k": dict(M=256, N=256, K=16384, dtype="f32", dist="uniform", op_b="N"),
    # one GPU's share of the 4096^3 problems split 8 ways by rows of A and C
    "m8_f16_shard": dict(M=512, N=4096, K=4096, dtype="f16", dist="uniform", op_b="N"),
    "m8_f32_shard": dict(M=512, N=4096, K=4096, dtype="f32", dist="uniform", op_b="N"),
    # four rounds of 256 output tiles of 256 x 256 (the persistent grid's case)
    "r4_f16_8192x8192x2048": dict(M=8192, N=8192, K=2048, dtype="f16", dist="uniform", op_b="N"),
    # 289 tiles of 256 x 256: one round of 256 and a tail of 33 (stream-K with a workspace)
    "t33_f16_4352x4352x2048": dict(M=4352, N=4352, K=2048, dtype="f16", dist="uniform", op_b="N"),
}


def make_config(name: str, seed: int = 0) -> Operands:
    c = CONFIGS[name] if name in CONFIGS else EXTRA_CONFIGS[name]
    return make_operands(c["M"], c["N"], c["K"], dtype=c["dtype"], dist=c["dist"], seed=seed, op_b=c["op_b"])
