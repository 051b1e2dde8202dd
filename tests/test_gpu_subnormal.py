"""Subnormal inputs and results are kept, not flushed to zero, on every kernel family.

A holds subnormal values of its type: integer multiples (1..63, random sign) of the
smallest subnormal, 2^-24 for fp16, 2^-133 for bf16, 2^-149 for fp32. B holds
integers in [-4, 4]. Every product and every partial sum is then a small integer
times that unit, exact in fp32 whatever the order of the sum (for fp32 and bf16
inputs the results are themselves fp32 subnormals or just above), so C must equal
the oracle's fp64 result bit for bit; a kernel that flushed subnormal inputs,
products or sums would return zeros.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi
import oracle

from gpu_util import check_untouched, run_ops

pytestmark = pytest.mark.gpu

UNIT = {"f16": 2.0 ** -24, "bf16": 2.0 ** -133, "f32": 2.0 ** -149}


def operands(M, N, K, dtype, op_b, seed):
    rng = np.random.default_rng(seed)
    a = rng.integers(1, 64, (M, K)).astype(np.float32) * np.float32(UNIT[dtype])
    a *= np.where(rng.random((M, K)) < 0.5, -1, 1).astype(np.float32)
    b = rng.integers(-4, 5, (K, N)).astype(np.float32)
    return gi.from_values(a, b, dtype, op_b)


CASES = [
    ("simt-f32", "f32", "N", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_LDS)),
    ("simt-f16", "f16", "N", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_LDS)),
    ("simt-bf16-T", "bf16", "T", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_LDS)),
    ("mfma-f32", "f32", "N", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_MFMA, schedule=1)),
    ("mfma-f16", "f16", "N", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_MFMA, schedule=1)),
    ("mfma-bf16-T", "bf16", "T", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_MFMA, schedule=1)),
    ("three-stage-f32", "f32", "N", (300, 260, 200), dict(schedule=6)),
    ("ping-pong-f16", "f16", "N", (300, 264, 224), dict(schedule=2)),
    ("ping-pong-bf16-T", "bf16", "T", (300, 260, 224), dict(schedule=2)),
    ("pipelined8-f16", "f16", "N", (300, 264, 200), dict(schedule=5, threads=512)),
    ("pipelined4-bf16-T", "bf16", "T", (300, 260, 200), dict(schedule=5, threads=256)),
    ("pipelined-reg8-f16", "f16", "N", (300, 263, 203), dict(schedule=7, threads=512)),
    ("pipelined-reg4-bf16-T", "bf16", "T", (300, 261, 203), dict(schedule=7, threads=256)),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_subnormal_inputs_exact(case):
    name, dtype, op_b, (M, N, K), req = case
    print(f"subnormal case {name}: {M}x{N}x{K} {dtype} op {op_b}", flush=True)
    ops = operands(M, N, K, dtype, op_b, seed=7)
    Cfull = run_ops(ops, dg.request(**req))
    check_untouched(Cfull, M, N)
    Cref, _ = oracle.gemm_ref(ops, want_d=False)
    assert np.count_nonzero(Cref) > 0.9 * M * N
    assert np.array_equal(Cfull[:M, :N].astype(np.float64), Cref)
