"""Pins for the CPU oracle: checks against facts that do not come from the oracle itself.

Each pin is a function of a `ref(ops, rows=None) -> (Cref, D)` callable so that the
same checks can be run against deliberately broken builds of the oracle (see
test_oracle_mutants.py), which must fail at least one of them.

Pins:
  P1  exact rational sums (fractions.Fraction) on tiny integer and dyadic inputs,
      and a forward-error bound against exact sums on random fp32 inputs
  P2  identity matrices reproduce the other operand exactly (all layouts, padded ld)
  P3  permutation matrices permute rows / columns exactly
  P4  rank-1 closed form  (u x^T)(y v^T) = (x . y) u v^T
  P5  integer patterns: exact against Python integer arithmetic, every dtype
  P6  degenerate shapes (K = 0 gives zeros; M = 0 / N = 0 give empty results)
  P7  float64 library product (numpy) on random data, normalized difference <= 1e-13
  P8  the fp16 precision figures printed in "Shared memory and tensor cores" 13.8
  P9  the fp16 / bf16 decoders against numpy's own conversions, all 65536 patterns
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np
import pytest

import gemm_inputs as gi
import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def default_ref(ops, rows=None):
    return oracle.gemm_ref(ops, rows=rows)


def logical(ops):
    """Logical float64 A (M x K) and B (K x N) from storage, via numpy's own conversions."""
    def dec(x):
        if ops.dtype == "f32":
            return x.astype(np.float64)
        if ops.dtype == "f16":
            return x.view(np.float16).astype(np.float64)
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    a = dec(ops.A).reshape(ops.M, ops.lda)[:, : ops.K] if ops.M else np.zeros((0, ops.K))
    if ops.op_b == "N":
        b = dec(ops.B).reshape(ops.K, ops.ldb)[:, : ops.N] if ops.K else np.zeros((0, ops.N))
    else:
        b = dec(ops.B).reshape(ops.N, ops.ldb)[:, : ops.K].T if ops.N else np.zeros((ops.K, 0))
    return a, b


# ---------------------------------------------------------------- P1
def pin_fraction_exact(ref):
    rng = np.random.default_rng(11)
    for (M, N, K) in [(1, 1, 1), (2, 3, 5), (3, 2, 7), (5, 7, 3), (7, 5, 16), (16, 17, 33), (17, 16, 1)]:
        for dtype in ("f32", "f16", "bf16"):
            a = rng.integers(-8, 9, (M, K)).astype(np.float32) / 4.0     # dyadic, exact in all dtypes
            b = rng.integers(-8, 9, (K, N)).astype(np.float32) / 2.0
            for op_b in ("N", "T"):
                ops = gi.from_values(a, b, dtype, op_b)
                C, D = ref(ops)
                for i in range(M):
                    for j in range(N):
                        exact = sum(Fraction(float(a[i, k])) * Fraction(float(b[k, j])) for k in range(K))
                        dexact = sum(abs(Fraction(float(a[i, k])) * Fraction(float(b[k, j]))) for k in range(K))
                        assert Fraction(C[i, j]) == exact, (M, N, K, dtype, op_b, i, j)
                        assert Fraction(D[i, j]) == dexact, (M, N, K, dtype, op_b, i, j)


def pin_fraction_bound(ref):
    """Random fp32 inputs: |Cref - exact| <= gamma_K * D with gamma_K = K u / (1 - K u), u = 2^-53."""
    ops = gi.make_operands(9, 11, 37, "f32", "uniform", seed=3)
    C, D = ref(ops)
    a, b = logical(ops)
    K = ops.K
    u = Fraction(1, 2 ** 53)
    gamma = K * u / (1 - K * u)
    for i in range(ops.M):
        for j in range(ops.N):
            exact = sum(Fraction(a[i, k]) * Fraction(b[k, j]) for k in range(K))
            dex = sum(abs(Fraction(a[i, k]) * Fraction(b[k, j])) for k in range(K))
            assert abs(Fraction(C[i, j]) - exact) <= gamma * dex
            # D itself sums non-negative terms: relative error <= gamma
            assert abs(Fraction(D[i, j]) - dex) <= gamma * dex
            assert dex > 0


# ---------------------------------------------------------------- P2
def pin_identity(ref):
    for dtype in ("f32", "f16", "bf16"):
        for op_b in ("N", "T"):
            ops = gi.make_operands(13, 9, 13, dtype, "uniform", seed=5, op_b=op_b,
                                   lda=13 + 3, ldb=(9 + 2) if op_b == "N" else (13 + 4))
            _, b = logical(ops)
            eye = np.eye(13, dtype=np.float32)
            left = gi.Operands(13, 9, 13, dtype, op_b, 13, ops.ldb, gi.to_storage(eye, dtype).reshape(-1), ops.B)
            C, _ = ref(left)
            assert np.array_equal(C, b), (dtype, op_b)
            # B = I: C = A
            ops2 = gi.make_operands(6, 8, 8, dtype, "uniform", seed=6, lda=11)
            a2, _ = logical(ops2)
            right = gi.from_values(np.zeros((6, 8)), np.eye(8), dtype, op_b)
            right = gi.Operands(6, 8, 8, dtype, op_b, ops2.lda, right.ldb, ops2.A, right.B)
            C2, _ = ref(right)
            assert np.array_equal(C2, a2), (dtype, op_b)


# ---------------------------------------------------------------- P3
def pin_permutation(ref):
    rng = np.random.default_rng(7)
    for dtype in ("f32", "bf16"):
        for op_b in ("N", "T"):
            ops = gi.make_operands(10, 7, 10, dtype, "normal", seed=8, op_b=op_b)
            _, b = logical(ops)
            p = rng.permutation(10)
            P = np.zeros((10, 10), np.float32)
            P[np.arange(10), p] = 1.0                      # (P B)[i] = B[p[i]]
            left = gi.Operands(10, 7, 10, dtype, op_b, 10, ops.ldb, gi.to_storage(P, dtype).reshape(-1), ops.B)
            C, _ = ref(left)
            assert np.array_equal(C, b[p, :]), (dtype, op_b)
            # column permutation: A Q with Q[q[j], j] = 1 -> (A Q)[:, j] = A[:, q[j]]
            ops2 = gi.make_operands(5, 6, 6, dtype, "normal", seed=9)
            a2, _ = logical(ops2)
            q = rng.permutation(6)
            Q = np.zeros((6, 6), np.float32)
            Q[q, np.arange(6)] = 1.0
            rq = gi.from_values(np.zeros((5, 6)), Q, dtype, op_b)
            right = gi.Operands(5, 6, 6, dtype, op_b, ops2.lda, rq.ldb, ops2.A, rq.B)
            C2, _ = ref(right)
            assert np.array_equal(C2, a2[:, q]), (dtype, op_b)


# ---------------------------------------------------------------- P4
def pin_rank1(ref):
    # exact: small integers
    u = np.array([1, -2, 3, 0, 5], np.float32)
    x = np.array([2, 1, -1, 3], np.float32)
    y = np.array([1, -1, 2, 2], np.float32)
    v = np.array([3, 0, -2, 1, 1, -4], np.float32)
    a = np.outer(u, x)
    b = np.outer(y, v)
    s = float(x @ y)  # = 2 - 1 - 2 + 6 = 5
    assert s == 5.0
    for dtype in ("f32", "f16", "bf16"):
        for op_b in ("N", "T"):
            C, D = ref(gi.from_values(a, b, dtype, op_b))
            assert np.array_equal(C, s * np.outer(u, v).astype(np.float64))
            assert np.array_equal(D, float(np.abs(x) @ np.abs(y)) * np.abs(np.outer(u, v)).astype(np.float64))
    # random fp32 factors: within 1e-12 relative of the closed form evaluated in fp64
    rng = np.random.default_rng(12)
    K = 300
    u = rng.uniform(-1, 1, 7).astype(np.float32)
    v = rng.uniform(-1, 1, 9).astype(np.float32)
    x = rng.uniform(-1, 1, K).astype(np.float32)
    y = rng.uniform(-1, 1, K).astype(np.float32)
    a = np.outer(u, x).astype(np.float32)            # products rounded to fp32 here: use those values
    b = np.outer(y, v).astype(np.float32)
    C, D = ref(gi.from_values(a, b, "f32"))
    # closed form on the stored (rounded) factors: C_ij = sum_k a_ik b_kj; compare with
    # the rank-1 structure up to the fp32 rounding of a and b (|a - u x| <= 2^-24 |u x|)
    s = float(x.astype(np.float64) @ y.astype(np.float64))
    approx = s * np.outer(u.astype(np.float64), v.astype(np.float64))
    bound = 2.0 ** -22 * np.outer(np.abs(u), np.abs(v)) * float(np.abs(x).astype(np.float64) @ np.abs(y))
    assert np.all(np.abs(C - approx) <= bound + 1e-12 * D)


# ---------------------------------------------------------------- P5
def pin_integer_patterns(ref):
    for (M, N, K) in [(17, 19, 23), (33, 8, 64), (5, 40, 3)]:
        i = np.arange(M)[:, None]
        k = np.arange(K)[None, :]
        a = (((7 * i + 3 * k) % 7) - 3).astype(np.int64)
        kk = np.arange(K)[:, None]
        j = np.arange(N)[None, :]
        b = (((5 * kk + 2 * j + 1) % 7) - 3).astype(np.int64)
        exact = np.zeros((M, N), dtype=object)
        for ii in range(M):
            for jj in range(N):
                exact[ii, jj] = sum(int(a[ii, t]) * int(b[t, jj]) for t in range(K))
        for dtype in ("f32", "f16", "bf16"):
            for op_b in ("N", "T"):
                C, D = ref(gi.from_values(a.astype(np.float32), b.astype(np.float32), dtype, op_b))
                assert np.array_equal(C, exact.astype(np.float64)), (M, N, K, dtype, op_b)


# ---------------------------------------------------------------- P6
def pin_degenerate(ref):
    for dtype in ("f32", "bf16"):
        ops = gi.make_operands(4, 5, 0, dtype)
        C, D = ref(ops)
        assert C.shape == (4, 5) and not C.any() and not D.any()
        for (M, N) in [(0, 5), (4, 0), (0, 0)]:
            C, D = ref(gi.make_operands(M, N, 3, dtype))
            assert C.shape == (M, N)


# ---------------------------------------------------------------- P7
def pin_numpy_f64(ref):
    for dtype, op_b, (M, N, K) in [("f32", "N", (70, 50, 90)), ("f16", "T", (33, 65, 129)),
                                  ("bf16", "T", (31, 29, 257)), ("f32", "T", (8, 130, 40))]:
        ops = gi.make_operands(M, N, K, dtype, "normal", seed=21, op_b=op_b)
        a, b = logical(ops)
        C, D = ref(ops)
        Dn = np.abs(a) @ np.abs(b)
        assert np.max(np.abs(C - a @ b) / Dn) <= 1e-13
        assert np.max(np.abs(D - Dn) / Dn) <= 1e-13
    # the row-sampled interface returns exactly the same rows
    ops = gi.make_operands(40, 33, 21, "f32", "uniform", seed=2)
    Cf, Df = ref(ops)
    rows = np.array([39, 0, 17, 17, 5])
    Cs, Ds = ref(ops, rows=rows)
    assert np.array_equal(Cs, Cf[rows]) and np.array_equal(Ds, Df[rows])


# ---------------------------------------------------------------- P8
def _golden(name):
    out = {}
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            if line.startswith("#") or "|" not in line:
                continue
            parts = [p.strip() for p in line.split("|")]
            out[parts[0]] = parts[1:]
    return out


def pin_fp16_precision_13_8(ref):
    """Reproduce the three printed maximum errors of the chapter's fp16 precision model.

    The chapter's model: fp16 inputs, one 16x16x16 product per step accumulated in
    fp32, compared with an fp64 product of the fp32 originals, with an fp64 product
    of the fp16 inputs, and against an fp16-accumulated sum. Both fp64 references
    come from the oracle here (dtype f32 on the originals, dtype f16 on the rounded
    inputs); the tile loop and the fp16 accumulation are the chapter's models.
    """
    gold = _golden("fp16_precision_13_8.txt")
    M, N, K = 64, 32, 48
    o32 = gi.make_operands(M, N, K, "f32", "normal", seed=0)
    o16 = gi.make_operands(M, N, K, "f16", "normal", seed=0)
    A16 = o16.A.view(np.float16).reshape(M, K)
    B16 = o16.B.view(np.float16).reshape(K, N)
    sim = np.zeros((M, N), np.float32)
    for tm in range(M // 16):
        for tn in range(N // 16):
            c = np.zeros((16, 16), np.float32)
            for k0 in range(0, K, 16):
                a = A16[tm * 16:tm * 16 + 16, k0:k0 + 16].astype(np.float32)
                b = B16[k0:k0 + 16, tn * 16:tn * 16 + 16].astype(np.float32)
                c += a @ b
            sim[tm * 16:tm * 16 + 16, tn * 16:tn * 16 + 16] = c
    ref32, _ = ref(o32)
    ref16, _ = ref(o16)
    c16 = np.zeros((M, N), np.float16)
    for k in range(K):
        c16 = (c16 + (A16[:, k:k + 1] * B16[k:k + 1, :])).astype(np.float16)
    got = {
        "f16in_f32acc_vs_f64_of_f32_inputs": np.abs(sim - ref32).max(),
        "f16in_f32acc_vs_exact_f64_on_f16_inputs": np.abs(sim - ref16).max(),
        "f16in_f16acc_vs_f64_of_f32_inputs": np.abs(c16.astype(np.float64) - ref32).max(),
    }
    for key, (printed, decimals) in gold.items():
        assert f"{got[key]:.{int(decimals)}f}" == printed, (key, got[key], printed)


# ---------------------------------------------------------------- P9
def pin_decoders(_ref=None):
    bits = np.arange(65536, dtype=np.uint16)
    f16 = bits.view(np.float16).astype(np.float64)
    bf = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    # decode every pattern through the oracle's GEMM path: A = the patterns (1 x 65536), B = ones
    for dtype, want in (("f16", f16), ("bf16", bf)):
        finite = np.isfinite(want)
        sample = bits[finite]
        ops = gi.Operands(sample.size, 1, 1, dtype, "N", 1, 1, sample.copy(),
                          gi.to_storage(np.ones(1, np.float32), dtype))
        C, _ = oracle.gemm_ref(ops, want_d=False) if _ref is None else _ref(ops)
        assert np.array_equal(C[:, 0], want[finite]), dtype
        for b in (0x7C00, 0xFC00, 0x7E00, 0x7F80, 0xFF80, 0x7FC0):
            got = oracle.decode16(b, dtype)
            exp = (np.uint16(b).view(np.float16).astype(np.float64) if dtype == "f16"
                   else np.array([b << 16], np.uint32).view(np.float32).astype(np.float64)[0])
            assert (np.isnan(got) and np.isnan(exp)) or got == exp


PINS = [pin_fraction_exact, pin_fraction_bound, pin_identity, pin_permutation, pin_rank1,
        pin_integer_patterns, pin_degenerate, pin_numpy_f64, pin_fp16_precision_13_8]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_oracle_pin(pin):
    pin(default_ref)


def test_decoders():
    pin_decoders()


def test_opA_transposed_matches_rowmajor():
    """opA = column-major reads A(i,k) = A[k*lda + i]; same result as the row-major copy."""
    ops = gi.make_operands(12, 7, 9, "f32", "uniform", seed=4)
    a, _ = logical(ops)
    at = np.ascontiguousarray(a.T.astype(np.float32)).reshape(-1)
    opsT = gi.Operands(12, 7, 9, "f32", "N", 12, ops.ldb, at, ops.B)
    C1, D1 = oracle.gemm_ref(ops)
    C2, D2 = oracle.gemm_ref(opsT, op_a="T", lda=12)
    assert np.array_equal(C1, C2) and np.array_equal(D1, D2)


def test_check_criterion():
    from oracle.check import normalized_error
    Cref = np.array([[1.0, 0.0], [2.0, -1.0]])
    D = np.array([[2.0, 0.0], [4.0, 1.0]])
    assert normalized_error(Cref.astype(np.float32), Cref, D) == 0.0
    C = Cref.copy()
    C[1, 0] += 4e-5
    assert abs(normalized_error(C, Cref, D) - 1e-5) < 1e-12
    C = Cref.copy()
    C[0, 1] = 1e-30                                  # D == 0 requires an exact zero
    assert normalized_error(C, Cref, D) == float("inf")
    C = Cref.copy()
    C[1, 1] = np.nan
    assert normalized_error(C, Cref, D) == float("inf")


def test_thread_count_applies_to_one_call():
    """A call with an explicit thread count leaves later default calls on all threads,
    and the result does not depend on the thread count."""
    ops = gi.make_operands(40, 30, 20, "f32", "uniform", seed=5)
    before = oracle.max_threads()
    C1, D1 = oracle.gemm_ref(ops, nthreads=1)
    assert oracle.max_threads() == before
    C0, D0 = oracle.gemm_ref(ops)
    assert np.array_equal(C1, C0) and np.array_equal(D1, D0)


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("op_b", ["N", "T"])
def test_oracle_non_finite_inputs(dtype, op_b):
    """IEEE classes of sums of products with NaN and infinite factors, worked by hand:
    an infinity times zero is NaN, infinities of both signs in one sum give NaN, one
    infinite product makes the sum infinite with its sign, a NaN factor makes NaN."""
    inf, nan = np.inf, np.nan
    a = np.array([[inf, 1.0], [nan, 0.0], [1.0, 2.0], [-inf, 1.0], [3.0, -1.0]])
    b = np.array([[0.0, 1.0, 2.0], [1.0, -inf, 4.0]])
    want = np.array([[nan, nan, inf],       # inf*0 + 1;  inf*1 + (-inf);  inf*2 + 4
                     [nan, nan, nan],       # a NaN factor in every sum
                     [2.0, -inf, 10.0],     # 0 + 2;  1 + 2*(-inf);  2 + 8
                     [nan, -inf, -inf],     # -inf*0 + 1;  -inf*1 + (-inf);  -inf*2 + 4
                     [-1.0, inf, 2.0]])     # 0 - 1;  3 + (-1)(-inf);  6 - 4
    ops = gi.from_values(a, b, dtype, op_b)
    C, _ = oracle.gemm_ref(ops)
    assert np.array_equal(np.isnan(C), np.isnan(want))
    fin = ~np.isnan(want)
    assert np.array_equal(C[fin], want[fin])
