"""Calls from several host threads at once, each on its own stream.

The library's only shared state is the per-device (CU count, architecture) cache,
filled under a mutex; error strings are thread-local; workspaces belong to the
caller. Eight threads each issue a mix of calls (plain, split K or packing with
their own workspace, a fused epilogue) on their own stream, several times over,
while a ninth keeps making invalid calls. Every output must be bit-identical to the
same call made alone beforehand (the kernels are deterministic), and the invalid
calls must keep returning their own error status and message.
"""
from __future__ import annotations

import threading

import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi

from gpu_util import _torch, device_storage

pytestmark = pytest.mark.gpu

JOBS = [
    # (kind, dtype, op_b, (M, N, K), request kwargs)
    ("plain", "f16", "N", (1024, 1024, 512), {}),
    ("plain", "f32", "T", (600, 500, 300), {}),
    ("plain", "bf16", "T", (301, 257, 103), {}),
    ("workspace", "f32", "N", (256, 256, 4096), dict(split_k=8)),
    ("workspace", "bf16", "T", (300, 264, 203), dict(pack=2)),
    ("epilogue", "f16", "N", (512, 768, 256), {}),
    ("plain", "f16", "T", (2048, 512, 1024), dict(schedule=5)),
    ("plain", "f32", "N", (1024, 1024, 1024), {}),
]
WS = 1 << 25


class Job:
    def __init__(self, torch, idx, kind, dtype, op_b, shape, req):
        M, N, K = shape
        lda = K + (1 if kind == "workspace" and req.get("pack") else 0)
        ldb = (K if op_b == "T" else N) + (1 if kind == "workspace" and req.get("pack") else 0)
        ops = gi.make_operands(M, N, K, dtype, "normal", seed=80 + idx, op_b=op_b, lda=lda, ldb=ldb)
        self.kind, self.ops, self.req = kind, ops, dg.request(**req)
        self.At, self.a = device_storage(ops.A)
        self.Bt, self.b = device_storage(ops.B)
        out_dt = torch.bfloat16 if kind == "epilogue" else torch.float32
        self.C = torch.zeros(M * N, dtype=out_dt, device="cuda")
        self.W = torch.empty(WS // 4, dtype=torch.float32, device="cuda")
        self.bias = torch.randn(N, device="cuda")
        self.ep = dg.epilogue(alpha=0.75, bias=self.bias.data_ptr(), activation="gelu_tanh", out_dtype="bf16")

    def call(self, stream):
        o = self.ops
        args = (0, dg.OP_CODE[o.op_b], o.M, o.N, o.K, self.a, o.lda, self.b, o.ldb, self.C.data_ptr(), o.N,
                dg.DTYPE_CODE[o.dtype])
        if self.kind == "plain":
            dg.gemm_ex(*args, self.req, stream)
        elif self.kind == "workspace":
            dg.gemm_ex_workspace(*args, self.req, self.W.data_ptr(), WS, stream)
        else:
            dg.gemm_ex_epilogue(*args, self.ep, None, None, 0, stream)


def test_threads_and_streams():
    torch = _torch()
    jobs = [Job(torch, i, *j) for i, j in enumerate(JOBS)]
    # each call alone first
    expect = []
    for j in jobs:
        j.C.zero_()
        j.call(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        expect.append(j.C.clone())
        assert torch.isfinite(j.C.float()).all()
    streams = [torch.cuda.Stream() for _ in jobs]
    for j in jobs:
        j.C.fill_(float("nan"))
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(len(jobs) + 1)

    def worker(j, s):
        try:
            start.wait()
            for _ in range(5):
                j.call(s.cuda_stream)
        except Exception as e:  # reported below
            errors.append(repr(e))

    def invalid():
        try:
            start.wait()
            for i in range(200):
                st = dg.gemm(-1 - i, 16, 16, 0, 16, 0, 16, 0, 16, dg.GEMM_F32, check=False)
                msg = dg.gemm_last_error()
                if st != dg.GEMM_ERR_INVALID_VALUE or f"M = {-1 - i}," not in msg:
                    errors.append(f"call {i}: status {st}, message {msg!r}")
        except Exception as e:
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(j, s)) for j, s in zip(jobs, streams)]
    threads.append(threading.Thread(target=invalid))
    print(f"concurrency: {len(jobs)} calling threads and one making invalid calls", flush=True)
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors[:5]
    for i, (j, e) in enumerate(zip(jobs, expect)):
        assert torch.equal(j.C, e), f"job {i} ({j.kind}, {j.ops.dtype}) differs from its call alone"
