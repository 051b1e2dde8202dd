"""GPU parity of split-K products (gemm_ex_workspace) against the CPU oracle.

Every register-staged kernel of the menu runs with forced slice counts on ragged
shapes whose K spans several k-tiles; random data must meet the normalized
tolerance and integer-valued data must match bit for bit. The slices are added
in a fixed order, so repeated calls must agree bit for bit. The workspace is
prefilled with NaN: nothing read from it may leak into C.
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

DT_NAME = {0: "f32", 1: "f16", 2: "bf16"}


def _torch():
    import torch
    return torch


def _menu():
    import os
    return [e for e in dg.gemm_menu() if e["schedule"] == 1] if os.path.exists(dg.LIB_PATH) else []


SPLITTABLE = _menu()
IDS = [f"k{e['kernel_id']}-{'lds' if e['variant'] == 1 else 'mfma'}-{DT_NAME[e['dtype']]}-op{'NT'[e['opb']]}-"
       f"{'v16' if e['vec'] else 'v1'}-{e['bm']}x{e['bn']}-w{e['waves_m']}x{e['waves_n']}" for e in SPLITTABLE]


def run_split(ops: gi.Operands, cfg, ws_bytes=1 << 26, ldc=None, ws_fill=float("nan"), ws_offset=0):
    """C = A @ B through gemm_ex_workspace; returns (C storage incl. 2 extra rows, plan)."""
    torch = _torch()
    ldc = ldc or max(1, ops.N)
    rows = ops.M + 2
    At, a_ptr = device_storage(ops.A)
    Bt, b_ptr = device_storage(ops.B)
    Ct = torch.full((rows * ldc + 8,), float(SENTINEL), dtype=torch.float32, device="cuda")
    Wt = torch.full((ws_bytes // 4 + 8,), ws_fill, dtype=torch.float32, device="cuda")
    w_ptr = Wt.data_ptr() + ws_offset
    _, plan = dg.gemm_plan_workspace(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, ops.lda, ops.ldb, ldc,
                                     dg.DTYPE_CODE[ops.dtype], a_ptr, b_ptr, Ct.data_ptr(), 256, "gfx950", ws_bytes,
                                     cfg)
    print(f"split-K case M={ops.M} N={ops.N} K={ops.K} {ops.dtype} op {ops.op_b}: kernel {plan.kernel_id} "
          f"split {plan.split_k} chunk {plan.k_chunk}", flush=True)
    dg.gemm_ex_workspace(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, a_ptr, ops.lda, b_ptr, ops.ldb,
                         Ct.data_ptr(), ldc, dg.DTYPE_CODE[ops.dtype], cfg, w_ptr, ws_bytes,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = Ct[:rows * ldc].cpu().numpy().reshape(rows, ldc)
    return out, plan


def forced(e, split):
    return dg.request(variant=e["variant"], bm=e["bm"], bn=e["bn"], vec=e["vec"], waves_m=e["waves_m"],
                      waves_n=e["waves_n"], threads=e["threads"], schedule=1, split_k=split)


def shape_for(e):
    return e["bm"] + 37, e["bn"] + 19, 5 * e["bk"] + 13


def lds_for(e, M, N, K):
    dtype, op_b = DT_NAME[e["dtype"]], "NT"[e["opb"]]
    if e["vec"]:
        q = 4 if dtype == "f32" else 8
        return -(-(K + 1) // q) * q, -(-((N if op_b == "N" else K) + 1) // q) * q
    return K + 3, (N if op_b == "N" else K) + 5


@pytest.mark.parametrize("e", SPLITTABLE, ids=IDS)
def test_split_every_kernel(e):
    """Six k-tiles split into 3 slices (2 k-tiles each) on a ragged shape."""
    M, N, K = shape_for(e)
    lda, ldb = lds_for(e, M, N, K)
    ops = gi.make_operands(M, N, K, DT_NAME[e["dtype"]], "normal", seed=e["kernel_id"], op_b="NT"[e["opb"]],
                           lda=lda, ldb=ldb)
    C, plan = run_split(ops, forced(e, 3), ldc=N + 3)
    assert plan.split_k == 3 and plan.kernel_id == e["kernel_id"]
    check_untouched(C, M, N)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:M, :N], Cref, D) <= TOL[ops.dtype]


@pytest.mark.parametrize("dtype,op_b", [("f32", "N"), ("f16", "N"), ("bf16", "T"), ("f16", "T")])
@pytest.mark.parametrize("split", [2, 5, 8, 16])
def test_split_counts_integer_exact(dtype, op_b, split):
    """Integer data: every slice and the ordered sum are exact, so C equals the oracle."""
    M, N, K = 150, 133, 700
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k) % 7) - 3).astype(np.float32)
    kk = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    b = (((5 * kk + 2 * j + 1) % 7) - 3).astype(np.float32)
    ops = gi.from_values(a, b, dtype, op_b)
    C, plan = run_split(ops, dg.request(split_k=split), ldc=N + 1)
    assert plan.split_k > 1
    check_untouched(C, M, N)
    Cref, _ = oracle.gemm_ref(ops)
    assert np.array_equal(C[:M, :N].astype(np.float64), Cref)


def test_split_fewer_k_tiles_than_slices():
    ops = gi.make_operands(96, 80, 70, "f32", "uniform", seed=3)
    C, plan = run_split(ops, dg.request(split_k=8, variant=dg.GEMM_VARIANT_MFMA, bm=64, bn=64))
    assert plan.split_k == 3
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:96, :80], Cref, D) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_split_heuristic_long_k(dtype):
    """Few output tiles and a long K: the heuristic splits; results are reproducible
    call to call (fixed reduction order) whatever the workspace held before."""
    ops = gi.make_operands(256, 256, 16384, dtype, "uniform", seed=9)
    C1, plan = run_split(ops, None)
    C2, _ = run_split(ops, None, ws_fill=0.0)
    assert plan.split_k > 1
    assert np.array_equal(C1, C2)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C1[:256, :256], Cref, D) <= TOL[dtype]


def test_split_long_k_benchmark_problem():
    ops = gi.make_config("k1_f32_long_k")
    C, plan = run_split(ops, None)
    assert plan.split_k > 1
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:ops.M, :ops.N], Cref, D) <= TOL["f32"]


def test_split_small_workspace_falls_back():
    """Auto planning with too little workspace does not split, and is still correct."""
    ops = gi.make_operands(256, 256, 256, "f32", "uniform", seed=5)
    C, plan = run_split(ops, None, ws_bytes=1024)
    assert plan.split_k == 1
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:256, :256], Cref, D) <= TOL["f32"]


@pytest.mark.parametrize("schedule,waves_n", [(5, 4), (5, 2), (7, 4), (7, 2)])
@pytest.mark.parametrize("dtype,op_b", [("f16", "N"), ("bf16", "T")])
@pytest.mark.parametrize("split", [2, 3, 5])
def test_split_software_pipelined(schedule, waves_n, dtype, op_b, split):
    """The one-tile form of the software-pipelined kernels with K in slices of whole
    k-tiles, on edge tiles in M and N; K leaves a partial last k-tile in the last slice
    (a multiple of 8 for the direct copies, any for the register-staged form, whose
    operands here sit at 2-byte offsets)."""
    M, N = 300, 264 if op_b == "N" else 263
    if schedule == 5:
        K, lda, ldb = 32 * 9 + 8, None, None
        off = 0
    else:
        K = 32 * 9 + 5
        lda, ldb = K + 1, (N if op_b == "N" else K) + 3
        off = 1
    ops = gi.make_operands(M, N, K, dtype, "normal", seed=split + 10 * schedule + waves_n, op_b=op_b, lda=lda,
                           ldb=ldb)
    C, plan = run_split_offset(ops, dg.request(schedule=schedule, waves_n=waves_n, split_k=split), off, ldc=N + 3)
    assert plan.split_k == split and plan.schedule == schedule
    check_untouched(C, M, N)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:M, :N], Cref, D) <= TOL[dtype]


@pytest.mark.parametrize("schedule", [5, 7])
@pytest.mark.parametrize("op_b", ["N", "T"])
def test_split_software_pipelined_integer_exact(schedule, op_b):
    """Integer data through four slices of the software-pipelined kernel: bit-exact,
    and a second call gives the same bits."""
    M, N, K = 512, 256, 32 * 10
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k) % 7) - 3).astype(np.float32)
    b = (((5 * np.arange(K)[:, None] + 2 * np.arange(N)[None, :] + 1) % 7) - 3).astype(np.float32)
    ops = gi.from_values(a, b, "f16", op_b)
    req = dg.request(schedule=schedule, waves_n=4, split_k=4)
    C1, plan = run_split(ops, req, ldc=N + 1)
    C2, _ = run_split(ops, req, ldc=N + 1)
    assert plan.split_k == 4 and plan.schedule == schedule
    Cref, _ = oracle.gemm_ref(ops, want_d=False)
    assert np.array_equal(C1[:M, :N].astype(np.float64), Cref)
    assert np.array_equal(C1, C2)


def run_split_offset(ops, cfg, off, ldc):
    """run_split with operands placed `off` elements past an aligned address (the
    register-staged form's element-aligned rows)."""
    if off == 0:
        return run_split(ops, cfg, ldc=ldc)
    torch = _torch()
    rows = ops.M + 2
    tdt = torch.float16 if ops.dtype == "f16" else torch.bfloat16
    At = torch.from_numpy(np.concatenate([np.zeros(off, np.uint16), ops.A.astype(np.uint16)]).view(np.int16)).cuda()
    Bt = torch.from_numpy(np.concatenate([np.zeros(off, np.uint16), ops.B.astype(np.uint16)]).view(np.int16)).cuda()
    a_ptr, b_ptr = At.data_ptr() + 2 * off, Bt.data_ptr() + 2 * off
    Ct = torch.full((rows * ldc + 8,), float(SENTINEL), dtype=torch.float32, device="cuda")
    ws = 1 << 26
    Wt = torch.full((ws // 4 + 8,), float("nan"), dtype=torch.float32, device="cuda")
    _, plan = dg.gemm_plan_workspace(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, ops.lda, ops.ldb, ldc,
                                     dg.DTYPE_CODE[ops.dtype], a_ptr, b_ptr, Ct.data_ptr(), 256, "gfx950", ws, cfg)
    print(f"split-K case M={ops.M} N={ops.N} K={ops.K} {ops.dtype} op {ops.op_b} offset {off}: kernel "
          f"{plan.kernel_id} schedule {plan.schedule} split {plan.split_k}", flush=True)
    dg.gemm_ex_workspace(0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, a_ptr, ops.lda, b_ptr, ops.ldb,
                         Ct.data_ptr(), ldc, dg.DTYPE_CODE[ops.dtype], cfg, Wt.data_ptr(), ws,
                         torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    del tdt
    return Ct[:rows * ldc].cpu().numpy().reshape(rows, ldc), plan


@pytest.mark.parametrize("schedule,bm", [(8, 64), (9, 256), (9, 128)])
@pytest.mark.parametrize("op_b", ["N", "T"])
@pytest.mark.parametrize("split", [2, 3, 5])
def test_split_f32_direct_copy(schedule, bm, op_b, split):
    """The fp32 direct-copy tiles with K in slices of whole k-tiles (pairs for the 64 x 64
    tile, whose two K groups share each slice), on edge tiles in M and N."""
    M, N = 2 * bm + 37, 300 if op_b == "N" else 301
    K = 64 * 11
    ops = gi.make_operands(M, N, K, "f32", "normal", seed=split + schedule + bm, op_b=op_b)
    C, plan = run_split(ops, dg.request(schedule=schedule, bm=bm, split_k=split), ldc=N + 3)
    # slices of whole k-tile pairs on the 64 x 64 tile: 22 k-tiles asked for in five
    # slices become four of six
    assert (plan.split_k == split or (schedule == 8 and 2 <= plan.split_k < split)) and plan.schedule == schedule
    assert plan.bm == bm and (schedule != 8 or plan.k_chunk % 64 == 0)
    check_untouched(C, M, N)
    Cref, D = oracle.gemm_ref(ops)
    assert normalized_error(C[:M, :N], Cref, D) <= TOL["f32"]


@pytest.mark.parametrize("schedule,bm", [(8, 64), (9, 256), (9, 128)])
def test_split_f32_direct_copy_integer_exact(schedule, bm):
    """Integer data through four slices of the fp32 direct-copy tiles: bit-exact."""
    M, N, K = 300, 260, 64 * 12
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k) % 7) - 3).astype(np.float32)
    b = (((5 * np.arange(K)[:, None] + 2 * np.arange(N)[None, :] + 1) % 7) - 3).astype(np.float32)
    ops = gi.from_values(a, b, "f32", "N")
    C, plan = run_split(ops, dg.request(schedule=schedule, bm=bm, split_k=4), ldc=N + 1)
    assert plan.split_k == 4 and plan.schedule == schedule
    Cref, _ = oracle.gemm_ref(ops, want_d=False)
    assert np.array_equal(C[:M, :N].astype(np.float64), Cref)
