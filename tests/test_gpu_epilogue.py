"""GPU parity of fused epilogues (gemm_ex_epilogue) against the CPU oracle.

C = act(alpha * (A @ B) + beta * R + bias), stored as fp32, fp16 or bf16, through
every path that can run an epilogue: the register-staged MFMA kernel, the LDS
kernel, the ping-pong kernel on whole tiles, packed operands and split K. The
reference is oracle.epilogue over the oracle's exact product; the criterion is
oracle.check.epilogue_error. Outputs are prefilled with a sentinel (a bit pattern
for 16-bit outputs) that must survive outside C[:M, :N].
"""
from __future__ import annotations

import numpy as np
import pytest

import dense_gemm_06_amd as dg
import gemm_inputs as gi
import oracle
from oracle.check import epilogue_error
from oracle.epilogue import epilogue_ref

from gpu_util import device_storage

pytestmark = pytest.mark.gpu

SENT16 = 0x7BCD            # an fp16 / bf16 bit pattern no test writes
SENT32 = np.float32(-7.75e30)


def _torch():
    import torch
    return torch


def decode_out(bits_or_vals: np.ndarray, out: str) -> np.ndarray:
    if out == "f32":
        return bits_or_vals.astype(np.float64)
    u = bits_or_vals.astype(np.uint16)
    if out == "f16":
        return u.view(np.float16).astype(np.float64)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode_out(vals: np.ndarray, out: str) -> np.ndarray:
    """Values representable in `out` -> storage (float32 or uint16 bits)."""
    return gi.to_storage(np.asarray(vals, dtype=np.float32), out)


class Out:
    """An output (and optional residual) buffer of M x ldc in the output type."""

    def __init__(self, M, N, ldc, out, init=None):
        torch = _torch()
        self.M, self.N, self.ldc, self.out = M, N, ldc, out
        rows = M + 2
        if out == "f32":
            self.t = torch.full((rows * ldc + 8,), float(SENT32), dtype=torch.float32, device="cuda")
        else:
            self.t = torch.full((rows * ldc + 8,), SENT16 - 65536 if SENT16 > 32767 else SENT16, dtype=torch.int16,
                                device="cuda")
        if init is not None:  # init: M x N storage values placed in the rows
            host = self.t.cpu().numpy()
            view = host[:M * ldc].reshape(M, ldc)
            view[:, :N] = init.view(np.int16) if out != "f32" else init
            self.t.copy_(torch.from_numpy(host))
        self.ptr = self.t.data_ptr()

    def values(self):
        raw = self.t.cpu().numpy()
        if self.out != "f32":
            raw = raw.view(np.uint16)
        full = raw[:(self.M + 2) * self.ldc].reshape(self.M + 2, self.ldc)
        return full

    def check_untouched(self):
        full = self.values()
        sent = SENT32 if self.out == "f32" else np.uint16(SENT16)
        assert np.all(full[:self.M, self.N:] == sent) and np.all(full[self.M:, :] == sent), "write outside C"


def run_epi(ops: gi.Operands, out: str, alpha=1.25, beta=-0.5, act="gelu_tanh", with_bias=True, cfg=None,
            ws_bytes=0, in_place=False, seed=0, R_vals=None, bias_vals=None):
    """Run gemm_ex_epilogue; return (C values fp64 M x N, reference, Dp, plan)."""
    torch = _torch()
    M, N = ops.M, ops.N
    ldc = N + 3
    rng = np.random.default_rng(1000 + seed)
    if R_vals is None:
        R_vals = rng.standard_normal((M, N)).astype(np.float32)
    R_store = encode_out(R_vals, out)
    R_dec = decode_out(R_store, out)
    if bias_vals is None:
        bias_vals = rng.standard_normal(N).astype(np.float32)
    bias_t = torch.from_numpy(np.ascontiguousarray(bias_vals, dtype=np.float32)).cuda() if with_bias else None
    At, a_ptr = device_storage(ops.A)
    Bt, b_ptr = device_storage(ops.B)
    if in_place:
        Cb = Out(M, N, ldc, out, init=R_store)
        r_ptr, ldr = Cb.ptr, ldc
    else:
        Cb = Out(M, N, ldc, out)
        Rb = Out(M, N, N + 1, out, init=R_store)
        r_ptr, ldr = Rb.ptr, N + 1
    epi = dg.epilogue(alpha=alpha, beta=beta, R=r_ptr if beta != 0 else None, ldr=ldr if beta != 0 else 0,
                      bias=bias_t.data_ptr() if with_bias else None, activation=act, out_dtype=out)
    W = torch.empty(max(ws_bytes, 16) // 4 + 4, dtype=torch.float32, device="cuda")
    _, plan = dg.gemm_plan_workspace(0, dg.OP_CODE[ops.op_b], M, N, ops.K, ops.lda, ops.ldb, ldc,
                                     dg.DTYPE_CODE[ops.dtype], a_ptr, b_ptr, Cb.ptr, 256, "gfx950", ws_bytes, cfg,
                                     epi=epi)
    print(f"epilogue case M={M} N={N} K={ops.K} {ops.dtype}->{out} act {act} alpha {alpha} beta {beta} "
          f"in_place {in_place}: kernel {plan.kernel_id} schedule {plan.schedule} split {plan.split_k} "
          f"pack {plan.pack}", flush=True)
    dg.gemm_ex_epilogue(0, dg.OP_CODE[ops.op_b], M, N, ops.K, a_ptr, ops.lda, b_ptr, ops.ldb, Cb.ptr, ldc,
                        dg.DTYPE_CODE[ops.dtype], epi, cfg, W.data_ptr() if ws_bytes else None, ws_bytes,
                        torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    Cb.check_untouched()
    got = decode_out(Cb.values()[:M, :N], out)
    Cref, D = oracle.gemm_ref(ops)
    ref, Dp = epilogue_ref(Cref, D, alpha=alpha, beta=beta, R=R_dec if beta != 0 else None,
                           bias=bias_vals.astype(np.float64) if with_bias else None, act=act)
    return got, ref, Dp, plan


PATHS = {
    "mfma": dict(cfg=None, ws=0),
    "lds": dict(cfg=dict(variant=dg.GEMM_VARIANT_LDS), ws=0),
    "packed": dict(cfg=dict(pack=2), ws=1 << 24),
    "split": dict(cfg=dict(split_k=3), ws=1 << 24),
}


@pytest.mark.parametrize("path", list(PATHS))
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("out,act", [("f32", "gelu_tanh"), ("f16", "relu"), ("bf16", "none"), ("f32", "relu")])
def test_epilogue_paths(path, dtype, out, act):
    ops = gi.make_operands(150, 130, 150, dtype, "normal", seed=7, op_b="T" if dtype == "bf16" else "N",
                           lda=150 + 3, ldb=(130 if dtype != "bf16" else 150) + 5)
    p = PATHS[path]
    cfg = dg.request(**p["cfg"]) if p["cfg"] else None
    got, ref, Dp, plan = run_epi(ops, out, act=act, cfg=cfg, ws_bytes=p["ws"])
    if path == "packed":
        assert plan.pack == 2
    if path == "split":
        assert plan.split_k == 3
    assert epilogue_error(got, ref, Dp, dtype, out) <= 1.0


@pytest.mark.parametrize("schedule,waves_n", [(2, 0), (5, 2), (5, 4), (7, 2), (7, 4)])
@pytest.mark.parametrize("dtype,op_b", [("f16", "N"), ("bf16", "T")])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_epilogue_whole_tile_kernels(schedule, waves_n, dtype, op_b, out):
    """The LDS-staged epilogues of the ping-pong and software-pipelined kernels."""
    ops = gi.make_operands(512, 256, 96, dtype, "normal", seed=8, op_b=op_b)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh",
                                 cfg=dg.request(schedule=schedule, waves_n=waves_n))
    assert plan.schedule == schedule
    assert epilogue_error(got, ref, Dp, dtype, out) <= 1.0


@pytest.mark.parametrize("waves_n", [2, 4])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_epilogue_software_pipelined_edge_tiles(waves_n, out):
    """The staged epilogue of schedule 5 on edge tiles (M, N not multiples of 256)."""
    ops = gi.make_operands(300, 264, 96, "f16", "normal", seed=10)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", cfg=dg.request(schedule=5, waves_n=waves_n))
    assert plan.schedule == 5
    assert epilogue_error(got, ref, Dp, "f16", out) <= 1.0


@pytest.mark.parametrize("shape,dtype,op_b", [((300, 264, 96), "f16", "N"), ((513, 777, 96), "bf16", "T"),
                                              ((40, 8, 32), "bf16", "N"), ((600, 1, 128), "f16", "T")])
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_epilogue_ping_pong_edge_tiles(shape, dtype, op_b, out):
    """The LDS-staged epilogue of the ping-pong kernel (schedule 2) on edge tiles (M
    and N not multiples of 256; row-major B with N a multiple of 8): rows >= M and
    columns >= N of the staged tile must not be stored, with bias, GELU, a residual
    (beta != 0) and every output type."""
    M, N, K = shape
    ops = gi.make_operands(M, N, K, dtype, "normal", seed=M + N, op_b=op_b)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", cfg=dg.request(schedule=2))
    assert plan.schedule == 2 and plan.tiles_m == -(-M // 256) and plan.tiles_n == -(-N // 256)
    assert epilogue_error(got, ref, Dp, dtype, out) <= 1.0


@pytest.mark.parametrize("waves_n", [2, 4])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_epilogue_register_staged_sp_unaligned(waves_n, out):
    """Schedule 7's staged epilogue on an unaligned ragged problem (rows at 2-byte
    offsets, K and N not multiples of 8)."""
    ops = gi.make_operands(300, 263, 99, "bf16", "normal", seed=12, lda=101, ldb=267)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", cfg=dg.request(schedule=7, waves_n=waves_n))
    assert plan.schedule == 7
    assert epilogue_error(got, ref, Dp, "bf16", out) <= 1.0


@pytest.mark.parametrize("op_b", ["N", "T"])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_epilogue_f32_direct_copy(op_b, out):
    """The fp32 direct-copy tile (schedule 8) with a fused epilogue on edge tiles."""
    ops = gi.make_operands(300, 264 if op_b == "N" else 263, 128, "f32", "normal", seed=13, op_b=op_b)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", cfg=dg.request(schedule=8))
    assert plan.schedule == 8
    assert epilogue_error(got, ref, Dp, "f32", out) <= 1.0


@pytest.mark.parametrize("schedule", [5, 7])
@pytest.mark.parametrize("out", ["f32", "bf16", "f16"])
def test_epilogue_software_pipelined_split(schedule, out):
    """A K split of the software-pipelined kernel: the slices store plain partial
    products and the reduction applies alpha, beta R, bias and GELU."""
    ops = gi.make_operands(300, 264, 32 * 7 + 8, "f16", "normal", seed=21)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", ws_bytes=1 << 24,
                                 cfg=dg.request(schedule=schedule, waves_n=4, split_k=3))
    assert plan.schedule == schedule and plan.split_k == 3
    assert epilogue_error(got, ref, Dp, "f16", out) <= 1.0


@pytest.mark.parametrize("bm", [256, 128])
@pytest.mark.parametrize("op_b", ["N", "T"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_epilogue_f32_large_direct_copy(bm, op_b, out):
    """The fp32 large direct-copy tiles (schedule 9) with a fused epilogue on edge tiles."""
    ops = gi.make_operands(300, 264 if op_b == "N" else 263, 160, "f32", "normal", seed=17, op_b=op_b)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", cfg=dg.request(schedule=9, bm=bm))
    assert plan.schedule == 9 and plan.bm == bm
    assert epilogue_error(got, ref, Dp, "f32", out) <= 1.0


@pytest.mark.parametrize("op_b", ["N", "T"])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_epilogue_three_stage_fp32(op_b, out):
    """The fp32 three-stage schedule with a fused epilogue, ragged tiles."""
    ops = gi.make_operands(300, 200, 150, "f32", "normal", seed=9, op_b=op_b)
    got, ref, Dp, plan = run_epi(ops, out, act="gelu_tanh", cfg=dg.request(schedule=6))
    assert plan.schedule == 6
    assert epilogue_error(got, ref, Dp, "f32", out) <= 1.0


@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_epilogue_in_place(out):
    """R == C: the BLAS form C = alpha A B + beta C."""
    ops = gi.make_operands(100, 140, 64, "f32", "normal", seed=9)
    got, ref, Dp, _ = run_epi(ops, out, alpha=1.0, beta=0.75, act="none", with_bias=False, in_place=True)
    assert epilogue_error(got, ref, Dp, "f32", out) <= 1.0


def test_epilogue_k_zero():
    """K = 0: C = act(beta R + bias), A and B unread."""
    ops = gi.make_operands(33, 47, 0, "f16", "normal", seed=10)
    got, ref, Dp, _ = run_epi(ops, "f32", act="relu")
    assert epilogue_error(got, ref, Dp, "f16", "f32") <= 1.0


@pytest.mark.parametrize("out", ["f32", "f16"])
@pytest.mark.parametrize("path", ["mfma", "split"])
def test_epilogue_integer_exact(out, path):
    """Integer data, alpha 2, beta -1, integer R and bias, ReLU: every value is an
    integer below 2^11, exact in fp32 and fp16 whatever the order of operations."""
    M, N, K = 70, 90, 96
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    a = (((7 * i + 3 * k) % 3) - 1).astype(np.float32)
    kk = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    b = (((5 * kk + 2 * j + 1) % 3) - 1).astype(np.float32)
    ops = gi.from_values(a, b, "f16", "N")
    R_vals = ((np.arange(M)[:, None] + np.arange(N)[None, :]) % 7 - 3).astype(np.float32)
    bias_vals = (np.arange(N) % 11 - 5).astype(np.float32)
    p = PATHS[path]
    got, ref, _, _ = run_epi(ops, out, alpha=2.0, beta=-1.0, act="relu", cfg=dg.request(**p["cfg"]) if p["cfg"] else None,
                             ws_bytes=p["ws"], R_vals=R_vals, bias_vals=bias_vals)
    assert np.array_equal(got, ref)


def test_identity_epilogue_is_the_plain_store():
    """alpha 1, beta 0, no bias, no activation, fp32: bit-identical to gemm_ex."""
    torch = _torch()
    ops = gi.make_operands(130, 120, 70, "bf16", "normal", seed=11)
    got, ref, Dp, plan = run_epi(ops, "f32", alpha=1.0, beta=0.0, act="none", with_bias=False)
    At, a_ptr = device_storage(ops.A)
    Bt, b_ptr = device_storage(ops.B)
    C = torch.zeros((130, 123), dtype=torch.float32, device="cuda")
    dg.gemm_ex(0, 0, 130, 120, 70, a_ptr, ops.lda, b_ptr, ops.ldb, C.data_ptr(), 123, dg.GEMM_BF16, None,
               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(got, C.cpu().numpy()[:, :120].astype(np.float64))
