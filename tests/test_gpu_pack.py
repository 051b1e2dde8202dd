"""GPU parity of packed-operand products (gemm_ex_workspace with packing) against
the CPU oracle.

Packing copies A and B into zero-padded, aligned whole-tile buffers and runs the
product on those; C must hold exactly the M x N result and nothing else. The
workspace is prefilled with NaN, so padding the copy kernel failed to zero would
poison C. Unaligned bases and odd leading dimensions are the case packing is for.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi
import oracle
from oracle.check import TOL, normalized_error

from gpu_util import SENTINEL, check_untouched, device_storage

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


def run_ws(ops: gi.Operands, cfg, ws_bytes=1 << 27, ldc=None, a_off=0, b_off=0):
    torch = _torch()
    ldc = ldc or max(1, ops.N)
    rows = ops.M + 2
    At, a_ptr = device_storage(ops.A, a_off)
    Bt, b_ptr = device_storage(ops.B, b_off)
    Ct = torch.full((rows * ldc + 8,), float(SENTINEL), dtype=torch.float32, device="cuda")
    Wt = torch.full((ws_bytes // 4 + 8,), float("nan"), dtype=torch.float32, device="cuda")
    _, plan = dg.gemm_plan_workspace(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, ops.lda, ops.ldb, ldc,
                                     dg.DTYPE_CODE[ops.dtype], a_ptr, b_ptr, Ct.data_ptr(), 256, "gfx950", ws_bytes,
                                     cfg)
    print(f"packed case M={ops.M} N={ops.N} K={ops.K} {ops.dtype} op {ops.op_b} lda={ops.lda} ldb={ops.ldb}: "
          f"kernel {plan.kernel_id} schedule {plan.schedule} pack {plan.pack}", flush=True)
    dg.gemm_ex_workspace(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, a_ptr, ops.lda, b_ptr, ops.ldb,
                         Ct.data_ptr(), ldc, dg.DTYPE_CODE[ops.dtype], cfg, Wt.data_ptr(), ws_bytes,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return Ct[:rows * ldc].cpu().numpy().reshape(rows, ldc), plan


CASES = [(600, 300, 200), (257, 513, 95), (1, 256, 64), (300, 1, 33), (512, 256, 32)]


@pytest.mark.parametrize("dtype,op_b", [("f16", "N"), ("bf16", "T"), ("f16", "T"), ("bf16", "N")])
@pytest.mark.parametrize("schedule", [2, 4, 5, 1])  # schedule 5: the planner's 4- or 8-wave choice
@pytest.mark.parametrize("shape", CASES, ids=[f"{m}x{n}x{k}" for m, n, k in CASES])
def test_pack_onto_each_schedule(dtype, op_b, schedule, shape):
    """Odd leading dimensions and a base one element off 16 bytes: packing is the
    only way onto the aligned kernels."""
    M, N, K = shape
    ops = gi.make_operands(M, N, K, dtype, "normal", seed=M + N + K, op_b=op_b, lda=K + 1,
                           ldb=(N if op_b == "N" else K) + 3)
    C, plan = run_ws(ops, dg.request(pack=2, schedule=schedule), ldc=N + 5, a_off=1, b_off=3)
    assert plan.pack == 2 and plan.schedule == schedule and plan.vec == 1
    check_untouched(C, M, N)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:M, :N], Cref, D) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_pack_integer_exact(dtype):
    M, N, K = 333, 270, 301
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k + 2) % 7) - 3).astype(np.float32)
    kk = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    b = (((5 * kk + 2 * j + 1) % 7) - 3).astype(np.float32)
    ops = gi.from_values(a, b, dtype, "T", lda=K + 1, ldb=K + 1)
    C, plan = run_ws(ops, dg.request(pack=2), ldc=N + 1, a_off=1, b_off=1)
    assert plan.pack == 2
    check_untouched(C, M, N)
    Cref, _ = oracle.gemm_ref(ops)
    assert np.array_equal(C[:M, :N].astype(np.float64), Cref)


def test_pack_ragged_benchmark_problem():
    """The 3001 x 5003 x 1037 bf16 problem (column-major B, odd leading dimensions)
    packed (forced: the heuristic runs it directly on the register-staged
    software-pipelined kernel), every entry against the oracle."""
    ops = gi.make_config("c5_bf16_ragged")
    C, plan = run_ws(ops, dg.request(pack=2), ws_bytes=1 << 26)
    assert plan.pack == 2 and plan.schedule in (2, 5)   # two whole-tile kernels that measure the same here
    check_untouched(C, ops.M, ops.N)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:ops.M, :ops.N], Cref, D) <= TOL["bf16"]


def test_pack_not_used_for_aligned_whole_tiles():
    ops = gi.make_operands(512, 512, 256, "f16", "uniform", seed=4)
    C, plan = run_ws(ops, None)
    assert plan.pack == 1 and plan.vec == 1
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:512, :512], Cref, D) <= TOL["f16"]
