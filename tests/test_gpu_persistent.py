"""GPU parity of the persistent form of the software-pipelined kernel (schedule 5 with
a grid below the tile count) against the CPU oracle.

Each workgroup of the capped grid computes every grid-th output tile; the copies
of a tile's first three k-tiles run during the previous tile's last iterations and
the finished tile's epilogue goes through one LDS stage. These tests give each
workgroup several tiles (grids of 1, 3, 8, 16 and 23 workgroups), edge tiles in M
and N, both B layouts, both 16-bit input types, every small k-tile count the form
takes (4 and up) and a long K, integer data (bit-exact), a fused epilogue (also in
place, R = C) and the 4096^3 fp16 problem on grids of 64 and 192.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi
import oracle
from oracle.check import TOL, epilogue_error, normalized_error

from gpu_util import check_untouched, run_ops

pytestmark = pytest.mark.gpu


def plan_of(ops, req, ldc):
    st, plan = dg.gemm_plan(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, ops.lda, ops.ldb, ldc,
                            dg.DTYPE_CODE[ops.dtype], 1 << 30, 1 << 40, 1 << 41, 256, "gfx950", req)
    assert st == 0
    return plan


def run_persistent(ops, grid, ldc, **kw):
    req = dg.request(schedule=5, waves_n=4, max_grid=grid)
    plan = plan_of(ops, req, ldc)
    tiles = plan.tiles_m * plan.tiles_n
    print(f"persistent case M={ops.M} N={ops.N} K={ops.K} {ops.dtype} op {ops.op_b}: grid {plan.grid} of "
          f"{tiles} tiles, xcd_remap {plan.xcd_remap}", flush=True)
    assert plan.schedule == 5 and plan.threads == 512 and plan.grid == min(grid, tiles)
    return run_ops(ops, cfg=req, ldc=ldc, **kw), plan


SHAPES = [((1000, 1304, 256), "N"), ((1000, 1300, 256), "T"), ((769, 1025, 160), "T"), ((2048, 1536, 128), "N"),
          ((513, 2056, 384), "N")]


@pytest.mark.parametrize("grid", [1, 3, 8, 16, 23])
@pytest.mark.parametrize("shape,op_b", SHAPES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_persistent_grids(grid, shape, op_b, dtype):
    M, N, K = shape
    ops = gi.make_operands(M, N, K, dtype, "normal", seed=M + N + K + grid, op_b=op_b)
    C, plan = run_persistent(ops, grid, N + 3)
    check_untouched(C, M, N)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:M, :N], Cref, D) <= TOL[dtype]


@pytest.mark.parametrize("k_tiles", [4, 5, 6, 7, 8, 130])
@pytest.mark.parametrize("dtype,op_b", [("f16", "N"), ("bf16", "T")])
def test_persistent_k_tile_counts(k_tiles, dtype, op_b):
    """The copy stream crosses tiles in the last three iterations of each: with 4
    k-tiles every iteration but the first touches the next tile."""
    K = 32 * k_tiles
    ops = gi.make_operands(600, 776, K, dtype, "normal", seed=k_tiles, op_b=op_b)
    C, plan = run_persistent(ops, 5, ops.N + 4)
    check_untouched(C, ops.M, ops.N)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:ops.M, :ops.N], Cref, D) <= TOL[dtype]


@pytest.mark.parametrize("op_b", ["N", "T"])
def test_persistent_integer_exact(op_b):
    M, N, K = 1100, 1032, 1024
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k) % 7) - 3).astype(np.float32)
    b = (((5 * np.arange(K)[:, None] + 2 * np.arange(N)[None, :] + 1) % 7) - 3).astype(np.float32)
    ops = gi.from_values(a, b, "bf16", op_b)
    C, plan = run_persistent(ops, 7, N + 1)
    check_untouched(C, M, N)
    Cref, _ = oracle.gemm_ref(ops, want_d=False)
    assert np.array_equal(C[:M, :N].astype(np.float64), Cref)


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_persistent_fused_epilogue(in_place, out):
    from test_gpu_epilogue import run_epi
    ops = gi.make_operands(777, 1040, 256, "f16", "normal", seed=91, op_b="N")
    req = dg.request(schedule=5, waves_n=4, max_grid=6)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", cfg=req, in_place=in_place)
    assert plan.schedule == 5 and plan.grid == 6
    assert epilogue_error(got, ref, Dp, "f16", out) <= 1.0


@pytest.mark.parametrize("grid", [64, 192])
def test_persistent_c4_integer_exact(grid):
    """4096^3 fp16 integer data on a grid of 64 (four tiles per workgroup) or 192
    (one or two): every entry bit-exact."""
    M = N = K = 4096
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k) % 7) - 3).astype(np.float32)
    b = (((5 * np.arange(K)[:, None] + 2 * np.arange(N)[None, :] + 1) % 7) - 3).astype(np.float32)
    ops = gi.from_values(a, b, "f16")
    C, plan = run_persistent(ops, grid, N, extra_rows=0)
    Cref, _ = oracle.gemm_ref(ops, want_d=False)
    bad = np.argwhere(C.astype(np.float64) != Cref)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:5].tolist()}"


def test_persistent_benchmark_problem_full_size():
    """The 8192 x 8192 x 2048 fp16 problem (four rounds of 256 tiles) in the
    configuration the heuristic picks, which is the persistent grid of 256 that the
    benchmark times: every entry of C against the oracle."""
    ops = gi.make_config("r4_f16_8192x8192x2048")
    plan = plan_of(ops, None, ops.N)
    print(f"persistent benchmark problem: grid {plan.grid}, schedule {plan.schedule}", flush=True)
    assert plan.schedule == 5 and plan.grid == 256 and plan.tiles_m * plan.tiles_n == 1024
    C = run_ops(ops, ldc=ops.N, extra_rows=1)
    check_untouched(C, ops.M, ops.N)
    Cref, D = oracle.gemm_ref(ops)
    err = normalized_error(C[:ops.M, :ops.N], Cref, D)
    print(f"normalized error {err:.3e} over all {ops.M} x {ops.N} entries", flush=True)
    assert err <= TOL[ops.dtype], err
