"""GPU parity of grouped and strided-batched products against the CPU oracle.

A grouped call runs several independent C = A @ B in one persistent launch (the
README's grouped tile scheduler, section 8.4). Every problem of every call is
checked against the oracle on the same seeded inputs: random data within the
normalized tolerance, integer-valued data bit for bit. Each output buffer is
prefilled with a sentinel; everything outside the problems' C[:M, :N] regions
must keep it.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi
import oracle
from oracle.check import TOL, normalized_error

from gpu_util import SENTINEL, device_storage

pytestmark = pytest.mark.gpu


def _torch():
    import torch
    return torch


class Entry:
    """One gemm_problem entry: `batch` operand sets of one shape, placed at strides."""

    def __init__(self, members: list[gi.Operands], ldc: int, stride_a: int | None = None,
                 stride_b: int | None = None, stride_c: int | None = None, share_a=False, share_b=False):
        torch = _torch()
        m0 = members[0]
        self.members, self.M, self.N, self.K, self.ldc = members, m0.M, m0.N, m0.K, ldc
        self.batch = len(members)
        la, lb = len(m0.A), len(m0.B)
        self.sa = 0 if share_a else (stride_a if stride_a is not None else la + 3)
        self.sb = 0 if share_b else (stride_b if stride_b is not None else lb + 5)
        clen = max(self.M * ldc, 1)
        self.sc = stride_c if stride_c is not None else clen + 7
        self.clen = clen
        a = np.zeros((self.batch - 1) * self.sa + la + 8, dtype=m0.A.dtype)
        b = np.zeros((self.batch - 1) * self.sb + lb + 8, dtype=m0.B.dtype)
        for i, op in enumerate(members):
            a[i * self.sa:i * self.sa + la] = op.A
            b[i * self.sb:i * self.sb + lb] = op.B
        self.At, self.a_ptr = device_storage(a)
        self.Bt, self.b_ptr = device_storage(b)
        self.Ct = torch.full(((self.batch - 1) * self.sc + clen + 16,), float(SENTINEL), dtype=torch.float32,
                             device="cuda")
        self.c_ptr = self.Ct.data_ptr()

    def problem(self):
        m0 = self.members[0]
        return dg.problem(self.M, self.N, self.K, self.a_ptr, m0.lda, self.b_ptr, m0.ldb, self.c_ptr, self.ldc,
                          batch=self.batch, stride_a=self.sa, stride_b=self.sb, stride_c=self.sc)

    def check(self, exact=False):
        C = self.Ct.cpu().numpy()
        mask = np.ones(C.shape, dtype=bool)
        for i, op in enumerate(self.members):
            if self.M == 0 or self.N == 0:
                continue
            base = i * self.sc
            full = C[base:base + self.M * self.ldc].reshape(self.M, self.ldc)
            got = full[:, :self.N]
            rows = np.arange(self.M)[:, None] * self.ldc + np.arange(self.N)[None, :] + base
            mask[rows.ravel()] = False
            Cref, D = oracle.gemm_ref(op)
            if exact:
                assert np.array_equal(got.astype(np.float64), Cref), f"member {i}: not bit-exact"
            else:
                err = normalized_error(got, Cref, D)
                assert err <= TOL[op.dtype], (i, err)
        assert np.all(C[mask] == SENTINEL), "a grouped call wrote outside its outputs"


def run(entries: list[Entry], dtype: str, op_b: str, cfg=None):
    torch = _torch()
    probs = [e.problem() for e in entries]
    print(f"grouped call: {len(probs)} entries, dtype {dtype}, op {op_b}, "
          f"shapes {[(e.batch, e.M, e.N, e.K) for e in entries]}", flush=True)
    dg.gemm_grouped(dg.GEMM_OP_N, dg.OP_CODE[op_b], dg.DTYPE_CODE[dtype], probs, cfg,
                    torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()


def rand_entry(M, N, K, dtype, op_b, seed, batch=1, ld_pad=(0, 0, 0), **kw):
    members = []
    for i in range(batch):
        lda = max(1, K) + ld_pad[0]
        ldb = (max(1, N) if op_b == "N" else max(1, K)) + ld_pad[1]
        members.append(gi.make_operands(M, N, K, dtype, "normal", seed=seed * 100 + i, op_b=op_b, lda=lda, ldb=ldb))
    return Entry(members, ldc=max(1, N) + ld_pad[2], **kw)


def int_entry(M, N, K, dtype, op_b, seed):
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k + seed) % 7) - 3).astype(np.float32)
    kk = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    b = (((5 * kk + 2 * j + seed + 1) % 7) - 3).astype(np.float32)
    return Entry([gi.from_values(a, b, dtype, op_b)], ldc=N + 1)


def test_grouped_four_256_cubed_fp32():
    """The README's grouped workload: four 256^3 fp32 products in one launch."""
    entries = [Entry([gi.make_operands(256, 256, 256, "f32", "uniform", seed=s)], ldc=256) for s in range(4)]
    _, cfg = dg.gemm_grouped_plan(0, 0, dg.GEMM_F32, [e.problem() for e in entries])
    assert cfg.launches == 1 and cfg.tiles_total == 4 * cfg.tiles_m * cfg.tiles_n
    run(entries, "f32", "N")
    for e in entries:
        e.check()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("op_b", ["N", "T"])
def test_grouped_mixed_shapes(dtype, op_b):
    """Ragged shapes, a 1-row and a 1-column problem, K = 0, an empty problem and a batch."""
    entries = [
        rand_entry(300, 200, 100, dtype, op_b, 1, ld_pad=(3, 5, 2)),
        rand_entry(64, 64, 64, dtype, op_b, 2),
        rand_entry(1, 513, 7, dtype, op_b, 3),
        rand_entry(129, 1, 33, dtype, op_b, 4, ld_pad=(1, 1, 1)),
        rand_entry(77, 91, 0, dtype, op_b, 5),
        rand_entry(0, 50, 10, dtype, op_b, 6),
        rand_entry(100, 120, 80, dtype, op_b, 7, batch=3, ld_pad=(8, 8, 4)),
    ]
    run(entries, dtype, op_b)
    for e in entries:
        e.check()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_grouped_integer_exact(dtype):
    entries = [int_entry(M, N, K, dtype, op_b, s) for s, (M, N, K, op_b) in
               enumerate([(200, 136, 96, "N"), (33, 257, 65, "N"), (128, 128, 128, "N")])]
    run(entries, dtype, "N")
    for e in entries:
        e.check(exact=True)


def test_grouped_more_entries_than_one_launch_holds():
    """20 entries: the host splits them over two launches (16 segments each at most)."""
    rng = np.random.default_rng(11)
    entries = [rand_entry(int(rng.integers(1, 150)), int(rng.integers(1, 150)), int(rng.integers(1, 90)), "f16",
                          "N", 20 + i) for i in range(20)]
    _, cfg = dg.gemm_grouped_plan(0, 0, dg.GEMM_F16, [e.problem() for e in entries])
    assert cfg.launches == 2
    run(entries, "f16", "N")
    for e in entries:
        e.check()


@pytest.mark.parametrize("max_grid", [1, 3, 8])
def test_grouped_persistent_loop(max_grid):
    """A capped grid makes each workgroup walk many tiles of several problems."""
    entries = [rand_entry(256, 256, 256, "f32", "N", 40 + s) for s in range(3)] + \
              [rand_entry(130, 70, 300, "f32", "N", 44)]
    run(entries, "f32", "N", cfg=dg.request(max_grid=max_grid))
    for e in entries:
        e.check()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_grouped_lds_variant(dtype):
    entries = [rand_entry(150, 130, 70, dtype, "N", 50), rand_entry(64, 200, 33, dtype, "N", 51, batch=2)]
    run(entries, dtype, "N", cfg=dg.request(variant=dg.GEMM_VARIANT_LDS))
    for e in entries:
        e.check()


@pytest.mark.parametrize("dtype,op_b", [("bf16", "T"), ("f32", "N"), ("f16", "N")])
def test_strided_batched_shared_b(dtype, op_b):
    """Six problems with their own A and one shared B (stride_b = 0), padded strides."""
    torch = _torch()
    M, N, K = 96, 80, 72
    first = gi.make_operands(M, N, K, dtype, "normal", seed=60, op_b=op_b)
    members = [gi.make_operands(M, N, K, dtype, "normal", seed=61 + i, op_b=op_b) for i in range(6)]
    members = [gi.Operands(M, N, K, dtype, op_b, m.lda, m.ldb, m.A, first.B) for m in members]
    e = Entry(members, ldc=N + 4, share_b=True)
    print(f"strided batched: 6 x ({M}, {N}, {K}) {dtype} op {op_b}", flush=True)
    dg.gemm_strided_batched(0, dg.OP_CODE[op_b], M, N, K, e.a_ptr, members[0].lda, e.sa, e.b_ptr, members[0].ldb,
                            0, e.c_ptr, e.ldc, e.sc, 6, dg.DTYPE_CODE[dtype], None,
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    e.check()


@pytest.mark.parametrize("dtype", ["f32", "f16"])
def test_grouped_vector_path(dtype):
    """16-byte aligned bases, leading dimensions and strides give the 16-byte load path;
    so does an odd batch stride (16-byte loads from element-aligned addresses); the
    element-wise loads, forced, give the same result."""
    q = 4 if dtype == "f32" else 8
    aligned = [rand_entry(192, 160, 96, dtype, "N", 70, batch=2, stride_a=192 * 96 + 4 * q, stride_b=96 * 160 + q),
               rand_entry(64, 128, 64, dtype, "N", 71)]
    _, cfg = dg.gemm_grouped_plan(0, 0, dg.DTYPE_CODE[dtype], [e.problem() for e in aligned])
    assert cfg.vec == 1
    run(aligned, dtype, "N")
    for e in aligned:
        e.check()
    for vec in (-1, 0):
        unaligned = [rand_entry(192, 160, 93, dtype, "N", 72, batch=2, ld_pad=(1, 3, 0))]  # odd strides and lds
        _, cfg = dg.gemm_grouped_plan(0, 0, dg.DTYPE_CODE[dtype], [e.problem() for e in unaligned])
        assert cfg.vec == 1
        run(unaligned, dtype, "N", cfg=dg.request(vec=vec))
        unaligned[0].check()


# ---- grouped calls on the persistent software-pipelined kernel (schedule 5)

def aligned_entry(M, N, K, dtype, op_b, seed, batch=1, gap=8):
    """Rows and batch strides that are multiples of 16 bytes (8 elements)."""
    ldb = N if op_b == "N" else K
    members = [gi.make_operands(M, N, K, dtype, "normal", seed=seed * 100 + i, op_b=op_b, lda=K, ldb=ldb)
               for i in range(batch)]
    la, lb = len(members[0].A), len(members[0].B)
    up = lambda n: -(-n // 8) * 8 + gap
    return Entry(members, ldc=N + 3, stride_a=up(la), stride_b=up(lb))


SP = dg.request(schedule=5)  # forced: these are tests of the kernel, on shapes of any size


def sp_plan(entries, dtype, op_b, cfg=None):
    _, plan = dg.gemm_grouped_plan(0, dg.OP_CODE[op_b], dg.DTYPE_CODE[dtype], [e.problem() for e in entries],
                                   req=cfg)
    print(f"grouped plan: schedule {plan.schedule}, grid {plan.grid}, tiles {plan.tiles_total}", flush=True)
    return plan


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("op_b", ["N", "T"])
def test_grouped_software_pipelined_mixed(dtype, op_b):
    """Aligned problems of different M, N and K (whole k-tiles, four or more) in one
    persistent launch of the software-pipelined kernel: edge tiles, a batch, K from 128
    to 1056, the copy stream running on across problems."""
    entries = [
        aligned_entry(300, 264, 128, dtype, op_b, 1),
        aligned_entry(512, 512, 1056, dtype, op_b, 2),
        aligned_entry(257, 776, 160, dtype, op_b, 3, batch=3),
        aligned_entry(64, 8, 256, dtype, op_b, 4),
        aligned_entry(1000, 520, 224, dtype, op_b, 5),
    ]
    plan = sp_plan(entries, dtype, op_b, SP)
    assert plan.schedule == 5 and plan.threads == 512
    run(entries, dtype, op_b, cfg=SP)
    for e in entries:
        e.check()


@pytest.mark.parametrize("max_grid", [1, 3, 8, 16])
def test_grouped_software_pipelined_grids(max_grid):
    """Capped grids: each workgroup walks many tiles of several problems."""
    entries = [aligned_entry(512, 512, 256, "bf16", "T", 80 + s) for s in range(3)] + \
              [aligned_entry(300, 600, 128, "bf16", "T", 84, batch=2)]
    req = dg.request(schedule=5, max_grid=max_grid)
    plan = sp_plan(entries, "bf16", "T", req)
    assert plan.schedule == 5 and plan.grid == max_grid
    run(entries, "bf16", "T", cfg=req)
    for e in entries:
        e.check()


@pytest.mark.parametrize("op_b", ["N", "T"])
def test_grouped_software_pipelined_integer_exact(op_b):
    entries = []
    for s, (M, N, K) in enumerate([(300, 264, 256), (513, 520, 128), (256, 256, 512)]):
        i = np.arange(M)[:, None]
        k = np.arange(K)[None, :]
        a = (((7 * i + 3 * k + s) % 7) - 3).astype(np.float32)
        b = (((5 * np.arange(K)[:, None] + 2 * np.arange(N)[None, :] + s + 1) % 7) - 3).astype(np.float32)
        entries.append(Entry([gi.from_values(a, b, "f16", op_b)], ldc=N + 1))
    plan = sp_plan(entries, "f16", op_b, SP)
    assert plan.schedule == 5
    run(entries, "f16", op_b, cfg=SP)
    for e in entries:
        e.check(exact=True)


def test_strided_batched_software_pipelined():
    """Eight 768 x 1024 x 512 bf16 products with column-major B at padded strides."""
    torch = _torch()
    e = aligned_entry(768, 1024, 512, "bf16", "T", 90, batch=8, gap=64)
    m0 = e.members[0]
    plan = sp_plan([e], "bf16", "T", SP)
    assert plan.schedule == 5
    dg.gemm_strided_batched(0, dg.GEMM_OP_T, e.M, e.N, e.K, e.a_ptr, m0.lda, e.sa, e.b_ptr, m0.ldb, e.sb, e.c_ptr,
                            e.ldc, e.sc, e.batch, dg.GEMM_BF16, SP, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    e.check()
