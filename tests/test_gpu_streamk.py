"""GPU parity of the stream-K tail of the persistent software-pipelined kernel
(gemm_ex_workspace with stream_k = 2) against the CPU oracle.

The tiles that leave the last round of the grid partly idle (all tiles when there
are fewer of them than workgroups) are dealt out as equal k-tile shares to
sk_width workgroups ("Shared memory and tensor cores" section 13.10, split-K and
stream-K); shares that begin or end inside a tile leave partial sums in the
workspace, which a second launch adds in k order. The cases cover shares that
split tiles in two and in several pieces, shares moved to a tile boundary (those
that fall fewer than 4 k-tiles from one), empty shares, whole rounds before the
tail and none, edge tiles in M and N, both B layouts, both 16-bit input types,
integer data (bit-exact), a fused epilogue (also in place), bit-identical repeated
calls whatever the workspace held before, and a full-size problem on the grid of
256 the heuristic uses.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi
import oracle
from oracle.check import TOL, epilogue_error, normalized_error

from gpu_util import check_untouched
from test_gpu_splitk import run_split

pytestmark = pytest.mark.gpu

WS = 1 << 28


def sk_request(grid=0, width=0):
    return dg.request(schedule=5, waves_n=4, max_grid=grid, stream_k=2, sk_width=width)


def run_sk(ops, grid=0, width=0, ldc=None, ws_fill=float("nan")):
    req = sk_request(grid, width)
    C, plan = run_split(ops, req, ws_bytes=WS, ldc=ldc, ws_fill=ws_fill)
    tiles = plan.tiles_m * plan.tiles_n
    tail = tiles % plan.grid if tiles > plan.grid else tiles
    print(f"stream-K case M={ops.M} N={ops.N} K={ops.K} {ops.dtype} op {ops.op_b}: grid {plan.grid}, {tiles} "
          f"tiles, tail {tail} on {plan.sk_width} workgroups", flush=True)
    assert plan.stream_k == 2 and plan.schedule == 5 and plan.launches == 2
    if width:
        assert plan.sk_width == width
    return C, plan


# (M, N, K, op_b, grid, width): tails of 4 tiles over 5..8 workgroups (shares of 8-12
# k-tiles, some moved to a tile boundary), a tail behind two whole rounds, edge tiles,
# fewer tiles than workgroups (no whole round), and a share count where moved bounds
# leave some shares empty
CASES = [
    (768, 1024, 512, "N", 8, 8),
    (768, 1024, 512, "N", 8, 5),
    (768, 1024, 512, "T", 8, 7),
    (1000, 1000, 1024, "T", 12, 9),
    (1000, 1000, 1024, "T", 12, 12),
    (1280, 1544, 512, "N", 12, 12),
    (512, 512, 2048, "N", 0, 13),
    (512, 520, 2048, "T", 0, 64),
    (300, 776, 256, "N", 0, 12),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}x{c[1]}x{c[2]}{c[3]}-g{c[4]}-w{c[5]}" for c in CASES])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_streamk_parity(case, dtype):
    M, N, K, op_b, grid, width = case
    ops = gi.make_operands(M, N, K, dtype, "normal", seed=M + N + K + width, op_b=op_b)
    C, plan = run_sk(ops, grid, width, ldc=N + 3)
    check_untouched(C, M, N)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:M, :N], Cref, D) <= TOL[dtype]


@pytest.mark.parametrize("op_b", ["N", "T"])
def test_streamk_integer_exact_and_repeatable(op_b):
    """Integer data: every entry equals the oracle's exact sum; a second call over a
    workspace full of other values gives the same bits."""
    M, N, K = 1100, 1032, 1024
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k) % 7) - 3).astype(np.float32)
    b = (((5 * np.arange(K)[:, None] + 2 * np.arange(N)[None, :] + 1) % 7) - 3).astype(np.float32)
    ops = gi.from_values(a, b, "f16", op_b)
    C1, plan = run_sk(ops, grid=10, width=9, ldc=N + 1)
    check_untouched(C1, M, N)
    Cref, _ = oracle.gemm_ref(ops, want_d=False)
    assert np.array_equal(C1[:M, :N].astype(np.float64), Cref)
    C2, _ = run_sk(ops, grid=10, width=9, ldc=N + 1, ws_fill=123.0)
    assert np.array_equal(C1, C2)


def test_streamk_random_repeatable():
    """Random data: the fixup adds the partial sums in a fixed order, so repeated calls
    agree bit for bit."""
    ops = gi.make_operands(1000, 1000, 1024, "bf16", "normal", seed=5, op_b="T")
    C1, _ = run_sk(ops, grid=12, width=9)
    C2, _ = run_sk(ops, grid=12, width=9, ws_fill=-1.0)
    assert np.array_equal(C1, C2)


@pytest.mark.parametrize("in_place", [False, True])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_streamk_fused_epilogue(in_place, out):
    """alpha, beta * R, bias, GELU and the output type: applied by the product kernel
    to tiles one workgroup completes, and by the fixup to the split tiles."""
    from test_gpu_epilogue import run_epi
    ops = gi.make_operands(777, 1040, 512, "f16", "normal", seed=17, op_b="N")
    req = sk_request(grid=6, width=5)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", cfg=req, ws_bytes=WS, in_place=in_place)
    assert plan.stream_k == 2 and plan.grid == 6 and plan.sk_width == 5
    assert epilogue_error(got, ref, Dp, "f16", out) <= 1.0


@pytest.mark.parametrize("width", [0, 66, 256])
def test_streamk_full_size(width):
    """The 4352^2 x 2048 fp16 benchmark problem (289 tiles: one round of 256 and a tail
    of 33) on the grid of 256, the tail over the heuristic's width (0: what the
    benchmark times with a workspace), 66 or all 256 workgroups: every entry against
    the oracle."""
    ops = gi.make_config("t33_f16_4352x4352x2048")
    if width == 0:
        C, plan = run_split(ops, None, ws_bytes=WS)
        print(f"heuristic: stream_k {plan.stream_k}, width {plan.sk_width}", flush=True)
        assert plan.stream_k == 2
    else:
        C, plan = run_sk(ops, grid=0, width=width)
    assert plan.grid == 256
    check_untouched(C, ops.M, ops.N)
    Cref, D = oracle.gemm_ref(ops)
    err = normalized_error(C[:ops.M, :ops.N], Cref, D)
    print(f"normalized error {err:.3e} over all entries", flush=True)
    assert err <= TOL["f16"], err


def test_streamk_needs_workspace():
    """stream_k = 2 with too little workspace is refused before any launch."""
    ops = gi.make_operands(768, 1024, 512, "f16", "normal", seed=1, op_b="N")
    st, _ = dg.gemm_plan_workspace(0, 0, ops.M, ops.N, ops.K, ops.lda, ops.ldb, ops.N, dg.DTYPE_CODE["f16"],
                                   1 << 30, 1 << 40, 1 << 41, 256, "gfx950", 1 << 20, sk_request(8, 8), check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE
