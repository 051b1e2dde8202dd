"""gemm_ex_noalloc (the library's fixed scratch in place of a caller workspace)
against gemm_ex_workspace with a caller workspace of the same size, through the
C ABI: the planner sees the same workspace size, so both run the same kernels and
must give the same bits. Each case makes two calls in a row, the second on a
smaller problem, so the second runs on scratch that still holds the first call's
contents. One case packs the operands into the scratch, one splits K into it, one
keeps the partial sums of a stream-K tail in it, one uses neither; the first case
is also checked against the oracle.
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

WS = dg.GEMM_NOALLOC_SCRATCH_BYTES


def _run(ops, noalloc: bool, cfg=None):
    import torch
    ldc = ops.N + 3
    At, a_ptr = device_storage(ops.A)
    Bt, b_ptr = device_storage(ops.B)
    Ct = torch.full(((ops.M + 2) * ldc,), float(SENTINEL), dtype=torch.float32, device="cuda")
    s = torch.cuda.current_stream().cuda_stream
    args = (0, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, a_ptr, ops.lda, b_ptr, ops.ldb, Ct.data_ptr(), ldc,
            dg.DTYPE_CODE[ops.dtype])
    _, plan = dg.gemm_plan_workspace(*args[:5], ops.lda, ops.ldb, ldc, args[-1], a_ptr, b_ptr, Ct.data_ptr(),
                                     256, "gfx950", WS, cfg)
    if noalloc:
        dg.gemm_ex_noalloc(*args, cfg, s)
        W = None
    else:
        W = torch.full((WS // 4,), float("nan"), dtype=torch.float32, device="cuda")
        dg.gemm_ex_workspace(*args, cfg, W.data_ptr(), WS, s)
    torch.cuda.synchronize()
    out = Ct.cpu().numpy().reshape(ops.M + 2, ldc)
    del At, Bt, Ct, W
    return out, plan


CASES = {
    # rows that are not 16-byte aligned, packing forced: both operands are copied into
    # the scratch
    "packed": lambda: [gi.make_operands(3001, 5003, 1037, "bf16", "normal", seed=1, op_b="T", lda=1037, ldb=1037),
                       gi.make_operands(2500, 4000, 1037, "bf16", "normal", seed=2, op_b="T", lda=1039, ldb=1041)],
    # 16 output tiles facing a long K: split K into partial planes in the scratch
    "split": lambda: [gi.make_operands(256, 256, 16384, "f32", "uniform", seed=3),
                      gi.make_operands(128, 192, 8192, "f32", "uniform", seed=4)],
    # a stream-K tail on a persistent grid of 8 (12 and 12 tiles: tails of 4 over 5
    # workgroups): partial sums in the scratch
    "stream_k": lambda: [gi.make_operands(768, 1024, 512, "f16", "uniform", seed=7),
                         gi.make_operands(600, 1024, 384, "f16", "uniform", seed=8)],
    # neither (the scratch is not used)
    "plain": lambda: [gi.make_operands(1024, 1024, 512, "f16", "uniform", seed=5),
                      gi.make_operands(200, 136, 100, "f16", "uniform", seed=6)],
}


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_matches_workspace_call(name):
    for i, ops in enumerate(CASES[name]()):
        print(f"noalloc case {name} call {i}: M={ops.M} N={ops.N} K={ops.K} {ops.dtype} op {ops.op_b}", flush=True)
        cfg = (dg.request(pack=2) if name == "packed" else
               dg.request(schedule=5, waves_n=4, max_grid=8, stream_k=2, sk_width=5) if name == "stream_k" else None)
        got, plan = _run(ops, noalloc=True, cfg=cfg)
        ref, plan_ws = _run(ops, noalloc=False, cfg=cfg)
        assert plan.as_dict() == plan_ws.as_dict()
        if name == "packed":
            assert plan.pack == 2
        if name == "split" and i == 0:
            assert plan.split_k > 1
        if name == "stream_k":
            assert plan.stream_k == 2 and plan.sk_width == 5 and plan.grid == 8
        if name == "plain":
            assert plan.pack == 1 and plan.split_k == 1
        check_untouched(got, ops.M, ops.N)
        assert np.array_equal(got, ref), f"{np.sum(got != ref)} entries differ"
        if i == 0 and name == "packed":
            Cref, D = oracle.gemm_ref(ops)
            assert normalized_error(got[:ops.M, :ops.N], Cref, D) <= TOL[ops.dtype]


def test_noalloc_refuses_requests_beyond_the_scratch():
    """A forced split whose partial planes exceed the scratch is refused before any launch."""
    ops = gi.make_operands(2048, 2048, 4096, "f32", "uniform", seed=7)
    At, a_ptr = device_storage(ops.A)
    Bt, b_ptr = device_storage(ops.B)
    import torch
    C = torch.full((2048 * 2048,), 5.0, dtype=torch.float32, device="cuda")
    st = dg.gemm_ex_noalloc(0, 0, 2048, 2048, 4096, a_ptr, ops.lda, b_ptr, ops.ldb, C.data_ptr(), 2048, dg.GEMM_F32,
                            dg.request(split_k=4), torch.cuda.current_stream().cuda_stream, check=False)
    assert st == dg.GEMM_ERR_INVALID_VALUE
    assert "scratch" in dg.gemm_last_error()
    torch.cuda.synchronize()
    assert bool(torch.all(C == 5.0))
