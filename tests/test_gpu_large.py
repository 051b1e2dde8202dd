"""Operands past 2^31 elements, and leading dimensions at the library's limit.

The kernels add each tile's origin in 64-bit arithmetic and index inside a tile
with 32-bit per-lane offsets (at most 256 rows of a leading dimension below 2^23
elements). These cases put tile origins beyond 2^31 elements and per-lane offsets
just under 2^31, and check sampled output rows against the oracle.

The large operand is filled on the device (a seeded torch generator, normal values
rounded to the input type); the sampled rows are copied back bit for bit and handed
to the oracle as a problem of their own, so no host copy of the whole operand is
made. B comes from the shared seeded generator.
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi
import oracle
from oracle.check import TOL, normalized_error

from gpu_util import _torch, device_storage

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def fill_rows(torch, view, K, seed, chunk=1 << 18):
    """Normal values in the first K columns of every row of `view` (rows x ld)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for r0 in range(0, view.shape[0], chunk):
        r1 = min(view.shape[0], r0 + chunk)
        view[r0:r1, :K].copy_(torch.randn(r1 - r0, K, generator=g, device="cuda").to(view.dtype))


def host_bits(t):
    """A device tensor's elements as the flat storage array the oracle takes."""
    if t.dtype == _torch().float32:
        return t.contiguous().cpu().numpy().reshape(-1)
    return t.contiguous().view(_torch().int16).cpu().numpy().view(np.uint16).reshape(-1)


def sample(M, lda, tile=256, n_random=12, seed=0):
    """First and last rows, rows on both sides of the 2^31-element offset and of the
    tile boundary nearest to it, and random rows."""
    rng = np.random.default_rng(seed)
    rows = {0, 1, M - 2, M - 1}
    r31 = -(-(1 << 31) // lda)
    for r in (r31 - 1, r31, r31 + 1, r31 // tile * tile - 1, r31 // tile * tile, (r31 // tile + 1) * tile):
        if 0 <= r < M:
            rows.add(r)
    rows |= set(int(x) for x in rng.integers(0, M, n_random))
    return np.array(sorted(rows))


def check_large_a(M, N, K, dtype, lda, seed, expect_schedule=None, req=None):
    torch = _torch()
    tdt = getattr(torch, TORCH_DT[dtype])
    A = torch.empty(M * lda, dtype=tdt, device="cuda")
    fill_rows(torch, A.view(M, lda), K, seed)
    small = gi.make_operands(1, N, K, dtype, "normal", seed=seed)  # only its B is used
    Bt, b_ptr = device_storage(small.B)
    C = torch.empty(M * N, dtype=torch.float32, device="cuda")
    st, plan = dg.gemm_plan(0, 0, M, N, K, lda, small.ldb, N, dg.DTYPE_CODE[dtype], A.data_ptr(), b_ptr,
                            C.data_ptr(), 256, "gfx950", req)
    print(f"case large A: M={M} N={N} K={K} {dtype} lda={lda} ({M * lda} elements) kernel {plan.kernel_id} "
          f"schedule {plan.schedule}", flush=True)
    if expect_schedule is not None:
        assert plan.schedule == expect_schedule
    dg.gemm_ex(0, 0, M, N, K, A.data_ptr(), lda, b_ptr, small.ldb, C.data_ptr(), N, dg.DTYPE_CODE[dtype], req,
               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = sample(M, lda)
    idx = torch.from_numpy(rows).to("cuda")
    sub = gi.Operands(len(rows), N, K, dtype, "N", K, small.ldb,
                      host_bits(A.view(M, lda).index_select(0, idx)[:, :K]), small.B)
    got = C.view(M, N).index_select(0, idx).cpu().numpy()
    del A, C, Bt
    torch.cuda.empty_cache()
    Cref, D = oracle.gemm_ref(sub)
    assert normalized_error(got, Cref, D) <= TOL[dtype]


def test_register_staged_a_beyond_2_31_elements():
    """fp16, 2^21 + 37 rows of 1056: 2.2e9 elements of A, tile rows past 2^31."""
    check_large_a((1 << 21) + 37, 96, 1056, "f16", 1056, seed=31)


def test_whole_tile_kernel_a_beyond_2_31_elements():
    """The 8-wave software-pipelined kernel on whole tiles (requested: the heuristic
    prefers smaller tiles for this narrow C): 8448 x 2^18 fp16 A."""
    check_large_a(8448, 256, 1 << 18, "f16", 1 << 18, seed=32, expect_schedule=5,
                  req=dg.request(schedule=5, waves_n=4))


def test_three_stage_fp32_a_beyond_2_31_elements():
    """The fp32 three-stage tile (requested): 2^20 + 100 rows of 2048 (2.1e9 elements of A)."""
    check_large_a((1 << 20) + 100, 256, 2048, "f32", 2048, seed=33, expect_schedule=6,
                  req=dg.request(schedule=6))


def test_large_direct_copy_fp32_a_beyond_2_31_elements():
    """The fp32 256 x 128 direct-copy tile, the heuristic's choice here: 2^20 + 100
    rows of 2048 (2.1e9 elements of A), copy sources past 2^31 elements."""
    check_large_a((1 << 20) + 100, 256, 2048, "f32", 2048, seed=34, expect_schedule=9)


@pytest.mark.parametrize("dtype,op_b", [("f16", "N"), ("f32", "T")])
def test_leading_dimension_at_the_limit(dtype, op_b):
    """A leading dimension of 2^23 - 8 elements (the largest accepted, rounded to 16
    bytes) on A for row-major B, on B for column-major B: per-lane offsets of up to
    255 rows just under 2^31 elements."""
    torch = _torch()
    tdt = getattr(torch, TORCH_DT[dtype])
    M, N, K, big = 300, 260, 200, (1 << 23) - 8
    lda = big if op_b == "N" else K
    ldb = N if op_b == "N" else big
    A = torch.empty(M * lda, dtype=tdt, device="cuda")
    fill_rows(torch, A.view(M, lda), K, seed=41)
    brows = K if op_b == "N" else N
    bcols = N if op_b == "N" else K
    B = torch.empty(brows * ldb, dtype=tdt, device="cuda")
    fill_rows(torch, B.view(brows, ldb), bcols, seed=42)
    C = torch.empty(M * N, dtype=torch.float32, device="cuda")
    print(f"case leading dimension {big}: {dtype} op {op_b}", flush=True)
    dg.gemm_ex(0, dg.OP_CODE[op_b], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C.data_ptr(), N,
               dg.DTYPE_CODE[dtype], None, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    rows = np.array(sorted({0, 1, 127, 128, 255, 256, 257, M - 1}))
    idx = torch.from_numpy(rows).to("cuda")
    a_rows = host_bits(A.view(M, lda).index_select(0, idx)[:, :K])
    b_dense = host_bits(B.view(brows, ldb)[:, :bcols])
    sub = gi.Operands(len(rows), N, K, dtype, op_b, K, bcols, a_rows, b_dense)
    got = C.view(M, N).index_select(0, idx).cpu().numpy()
    del A, B, C
    torch.cuda.empty_cache()
    Cref, D = oracle.gemm_ref(sub)
    assert normalized_error(got, Cref, D) <= TOL[dtype]
