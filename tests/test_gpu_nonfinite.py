"""NaN and infinities in A and B reach C by the IEEE rules, on every kernel family.

Entry (i, j) of C is the sum of the K products A(i,k) B(k,j). Without overflow its
class does not depend on the order of the sum: NaN if some product is NaN (a NaN
factor, or an infinity times zero) or if infinite products of both signs meet;
otherwise an infinity of the sign of the infinite products if there are any;
otherwise finite. Each case plants NaN, infinities and exact zeros at fixed places
(including the last row, the last column and the last k, so that edge tiles and
partial k-tiles see them) into seeded normal operands, runs one forced
configuration, and requires the oracle's class at every entry of C[:M, :N], the
oracle's sign at every infinity, the usual tolerance on the finite entries, and
no write outside C[:M, :N]. Zero padding and masking must never pair a real
infinity with a padding zero inside C[:M, :N].
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi
import oracle
from oracle.check import TOL, normalized_error

from gpu_util import SENTINEL, _torch, check_untouched, device_storage, run_ops

pytestmark = pytest.mark.gpu

BITS = {  # NaN, +Inf, -Inf, +0 as stored
    "f16": (0x7E00, 0x7C00, 0xFC00, 0x0000),
    "bf16": (0x7FC0, 0x7F80, 0xFF80, 0x0000),
}


def special(dtype, which):
    i = ("nan", "inf", "-inf", "zero").index(which)
    if dtype == "f32":
        return np.float32((np.nan, np.inf, -np.inf, 0.0)[i])
    return np.uint16(BITS[dtype][i])


def plant(ops: gi.Operands):
    """NaN in A(5, 7) and A(M-1, K-1); +Inf in A(17, 3) with B(3, 60) = 0; -Inf in
    A(40, 11) and +Inf in B(11, 50); -Inf in B(K-1, N-1)."""
    M, N, K = ops.M, ops.N, ops.K

    def set_a(i, k, v):
        ops.A[i * ops.lda + k] = special(ops.dtype, v)

    def set_b(k, j, v):
        ops.B[(k * ops.ldb + j) if ops.op_b == "N" else (j * ops.ldb + k)] = special(ops.dtype, v)

    set_a(5, 7, "nan")
    set_a(M - 1, K - 1, "nan")
    set_a(17, 3, "inf")
    set_b(3, 60, "zero")
    set_a(40, 11, "-inf")
    set_b(11, 50, "inf")
    set_b(K - 1, N - 1, "-inf")
    return ops


def compare(Cfull, ops):
    M, N = ops.M, ops.N
    check_untouched(Cfull, M, N)
    C = Cfull[:M, :N].astype(np.float64)
    Cref, D = oracle.gemm_ref(ops)
    assert np.array_equal(np.isnan(C), np.isnan(Cref)), "NaN pattern differs from the oracle"
    inf = np.isinf(Cref)
    assert np.array_equal(np.isinf(C), inf), "infinity pattern differs from the oracle"
    assert np.array_equal(np.sign(C[inf]), np.sign(Cref[inf])), "sign of an infinity differs"
    fin = np.isfinite(Cref) & np.isfinite(D)
    assert fin.sum() > 0.5 * M * N
    assert normalized_error(C[fin], Cref[fin], D[fin]) <= TOL[ops.dtype]
    # the planted values really produced every class
    assert np.isnan(Cref).any() and (Cref == np.inf).any() and (Cref == -np.inf).any()


PLAIN = [
    # (id, dtype, op_b, (M, N, K), request)
    ("simt-f32", "f32", "N", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_LDS)),
    ("simt-f16-T", "f16", "T", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_LDS)),
    ("mfma-f32", "f32", "T", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_MFMA, schedule=1, bm=128, bn=128)),
    ("mfma-k-groups-f32", "f32", "N", (300, 260, 200), dict(schedule=1, bm=64, bn=64, threads=512)),
    ("three-stage-f32", "f32", "N", (300, 260, 200), dict(schedule=6)),
    ("three-stage-f32-T", "f32", "T", (300, 260, 200), dict(schedule=6)),
    ("mfma-f16", "f16", "N", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_MFMA, schedule=1)),
    ("mfma-bf16-T", "bf16", "T", (300, 260, 200), dict(variant=dg.GEMM_VARIANT_MFMA, schedule=1)),
    ("ping-pong-f16", "f16", "N", (300, 264, 224), dict(schedule=2)),
    ("ping-pong-bf16-T", "bf16", "T", (300, 260, 224), dict(schedule=2)),
    ("pipelined8-f16", "f16", "N", (300, 264, 200), dict(schedule=5, threads=512)),
    ("pipelined4-bf16-T", "bf16", "T", (300, 260, 200), dict(schedule=5, threads=256)),
    ("pipelined-reg8-f16", "f16", "N", (300, 263, 203), dict(schedule=7, threads=512)),
    ("pipelined-reg4-bf16-T", "bf16", "T", (300, 261, 203), dict(schedule=7, threads=256)),
]


@pytest.mark.parametrize("case", PLAIN, ids=[c[0] for c in PLAIN])
def test_non_finite_plain(case):
    name, dtype, op_b, (M, N, K), req = case
    ops = plant(gi.make_operands(M, N, K, dtype, "normal", seed=61, op_b=op_b))
    cfg = dg.request(**req)
    st, plan = dg.gemm_plan(0, dg.OP_CODE[op_b], M, N, K, ops.lda, ops.ldb, N, dg.DTYPE_CODE[dtype], 0x10000,
                            0x20000, 0x40000, 256, "gfx950", cfg)
    print(f"non-finite case {name}: kernel {plan.kernel_id} schedule {plan.schedule}", flush=True)
    compare(run_ops(ops, cfg), ops)


def run_workspace(ops, cfg, ws_bytes=1 << 26):
    torch = _torch()
    rows, ldc = ops.M + 2, ops.N
    At, a_ptr = device_storage(ops.A)
    Bt, b_ptr = device_storage(ops.B)
    Ct = torch.full((rows * ldc + 8,), float(SENTINEL), dtype=torch.float32, device="cuda")
    Wt = torch.full((ws_bytes // 4 + 8,), float("nan"), dtype=torch.float32, device="cuda")
    _, plan = dg.gemm_plan_workspace(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, ops.lda, ops.ldb, ldc,
                                     dg.DTYPE_CODE[ops.dtype], a_ptr, b_ptr, Ct.data_ptr(), 256, "gfx950", ws_bytes,
                                     cfg)
    print(f"non-finite workspace case M={ops.M} N={ops.N} K={ops.K} {ops.dtype} op {ops.op_b}: kernel "
          f"{plan.kernel_id} split {plan.split_k} pack {plan.pack}", flush=True)
    dg.gemm_ex_workspace(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, a_ptr, ops.lda, b_ptr, ops.ldb,
                         Ct.data_ptr(), ldc, dg.DTYPE_CODE[ops.dtype], cfg, Wt.data_ptr(), ws_bytes,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return Ct[:rows * ldc].cpu().numpy().reshape(rows, ldc), plan


def test_non_finite_split_k():
    """K in four slices reduced in a fixed order: the classes survive the reduction."""
    ops = plant(gi.make_operands(300, 260, 1000, "f32", "normal", seed=62))
    Cfull, plan = run_workspace(ops, dg.request(split_k=4))
    assert plan.split_k == 4
    compare(Cfull, ops)


@pytest.mark.parametrize("dtype,op_b,schedule", [("bf16", "T", 0), ("f16", "N", 0), ("bf16", "T", 5), ("f16", "N", 2)])
def test_non_finite_packed(dtype, op_b, schedule):
    """Odd leading dimensions, packed into zero-padded whole tiles first (then the
    heuristic's kernel, or a forced direct-copy one): the padding zeros meet only
    other padding or rows and columns that are not stored."""
    M, N, K = 300, 264, 203
    ops = plant(gi.make_operands(M, N, K, dtype, "normal", seed=63, op_b=op_b, lda=K + 1,
                                 ldb=(N + 1) if op_b == "N" else (K + 1)))
    Cfull, plan = run_workspace(ops, dg.request(pack=2, schedule=schedule))
    assert plan.pack == 2 and (schedule == 0 or plan.schedule == schedule)
    compare(Cfull, ops)
