"""The library's calls captured in a HIP graph.

Nothing on the launch path allocates, copies, sets memory or synchronizes, so a
call can be recorded once and replayed. Each case captures one call, then replays
it three times; before every replay the inputs are rewritten by ordinary eager
work, and after it the graph's output must be bit-identical to an eager call of
the same configuration on the same data (the kernels are deterministic: no
atomics, fixed reduction orders).
"""
from __future__ import annotations

import pytest

import dense_gemm_06_amd as dg

from gpu_util import _torch

pytestmark = pytest.mark.gpu

TORCH_DT = {"f32": "float32", "f16": "float16", "bf16": "bfloat16"}


def operands(torch, M, N, K, dtype, op_b, pad=(0, 0)):
    tdt = getattr(torch, TORCH_DT[dtype])
    lda = K + pad[0]
    ldb = (N if op_b == "N" else K) + pad[1]
    A = torch.zeros(M * lda, dtype=tdt, device="cuda")
    B = torch.zeros((K if op_b == "N" else N) * ldb, dtype=tdt, device="cuda")
    return A, lda, B, ldb


def refill(torch, t, seed):
    """Rewrite a tensor's contents in place (eager work between replays)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    t.copy_(torch.randn(t.numel(), generator=g, device="cuda").to(t.dtype))


def run_case(make_call, inputs, outputs):
    """make_call(out_index, stream) enqueues the call writing outputs[out_index]."""
    torch = _torch()
    for i, t in enumerate(inputs):
        refill(torch, t, 100 + i)
    make_call(1, torch.cuda.current_stream().cuda_stream)   # warm-up, outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        make_call(0, side.cuda_stream)
    for rep in range(3):
        for i, t in enumerate(inputs):
            refill(torch, t, 1000 * (rep + 1) + i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        make_call(1, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        assert torch.equal(outputs[0], outputs[1]), f"replay {rep} differs from the eager call"
        assert torch.isfinite(outputs[0].float()).all()


@pytest.mark.parametrize("case", ["pipelined_f16", "pipelined_reg_bf16", "three_stage_f32", "register_staged_bf16_T",
                                  "persistent_f16", "direct_copy_f32", "small_tile_f32"])
def test_plain_call_in_graph(case):
    torch = _torch()
    dtype, op_b, shape, req = {
        "pipelined_f16": ("f16", "N", (1000, 1024, 1064), dg.request(schedule=5)),
        "pipelined_reg_bf16": ("bf16", "T", (1001, 1023, 1037), dg.request(schedule=7)),
        "three_stage_f32": ("f32", "N", (600, 500, 300), dg.request(schedule=6)),
        "register_staged_bf16_T": ("bf16", "T", (301, 257, 103), None),
        "persistent_f16": ("f16", "N", (1000, 1304, 256), dg.request(schedule=5, waves_n=4, max_grid=7)),
        "direct_copy_f32": ("f32", "T", (1000, 900, 384), dg.request(schedule=8)),
        "small_tile_f32": ("f32", "N", (256, 256, 256), dg.request(bm=16, bn=64, threads=256, schedule=1)),
    }[case]
    M, N, K = shape
    A, lda, B, ldb = operands(torch, M, N, K, dtype, op_b, pad=(3, 5) if case in ("register_staged_bf16_T", "pipelined_reg_bf16") else (0, 0))
    C = [torch.zeros(M * N, dtype=torch.float32, device="cuda") for _ in range(2)]
    print(f"graph case {case}: {shape} {dtype} op {op_b}", flush=True)

    def call(i, s):
        dg.gemm_ex(0, dg.OP_CODE[op_b], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C[i].data_ptr(), N,
                   dg.DTYPE_CODE[dtype], req, s)

    run_case(call, [A, B], C)


@pytest.mark.parametrize("case", ["split_k", "split_k_pipelined_f16", "split_k_pipelined_reg_bf16", "packed",
                                  "stream_k_f16", "stream_k_bf16_T"])
def test_workspace_call_in_graph(case):
    torch = _torch()
    if case == "stream_k_f16":
        dtype, op_b, (M, N, K), pad = "f16", "N", (768, 1024, 512), (0, 0)
        req = dg.request(schedule=5, waves_n=4, max_grid=8, stream_k=2, sk_width=5)
    elif case == "stream_k_bf16_T":
        dtype, op_b, (M, N, K), pad = "bf16", "T", (1000, 1000, 1024), (0, 0)
        req = dg.request(schedule=5, waves_n=4, max_grid=12, stream_k=2, sk_width=9)
    elif case == "split_k":
        dtype, op_b, (M, N, K), req, pad = "f32", "N", (256, 256, 8192), dg.request(split_k=8), (0, 0)
    elif case == "split_k_pipelined_f16":
        dtype, op_b, (M, N, K), req, pad = "f16", "N", (512, 768, 4096), dg.request(schedule=5, split_k=4), (0, 0)
    elif case == "split_k_pipelined_reg_bf16":
        dtype, op_b, (M, N, K), req, pad = "bf16", "T", (300, 500, 2053), dg.request(schedule=7, split_k=3), (3, 5)
    else:
        dtype, op_b, (M, N, K), req, pad = "bf16", "T", (301, 257, 103), dg.request(pack=2), (3, 5)
    A, lda, B, ldb = operands(torch, M, N, K, dtype, op_b, pad)
    C = [torch.zeros(M * N, dtype=torch.float32, device="cuda") for _ in range(2)]
    ws = 1 << 24
    W = [torch.empty(ws // 4, dtype=torch.float32, device="cuda") for _ in range(2)]
    _, plan = dg.gemm_plan_workspace(0, dg.OP_CODE[op_b], M, N, K, lda, ldb, N, dg.DTYPE_CODE[dtype], A.data_ptr(),
                                     B.data_ptr(), C[0].data_ptr(), 256, "gfx950", ws, req)
    print(f"graph case {case}: split {plan.split_k} pack {plan.pack} stream-K {plan.stream_k} launches "
          f"{plan.launches}", flush=True)
    assert plan.launches == 2 and (plan.stream_k == 2) == case.startswith("stream_k")

    def call(i, s):
        dg.gemm_ex_workspace(0, dg.OP_CODE[op_b], M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C[i].data_ptr(), N,
                             dg.DTYPE_CODE[dtype], req, W[i].data_ptr(), ws, s)

    run_case(call, [A, B], C)


def test_epilogue_call_in_graph():
    torch = _torch()
    M, N, K = 300, 264, 96
    A, lda, B, ldb = operands(torch, M, N, K, "f16", "N")
    bias = torch.zeros(N, dtype=torch.float32, device="cuda")
    C = [torch.zeros(M * N, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    ep = dg.epilogue(alpha=0.5, bias=bias.data_ptr(), activation="gelu_tanh", out_dtype="bf16")
    print("graph case epilogue", flush=True)

    def call(i, s):
        dg.gemm_ex_epilogue(0, 0, M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C[i].data_ptr(), N, dg.GEMM_F16,
                            ep, None, None, 0, s)

    run_case(call, [A, B, bias], C)


@pytest.mark.parametrize("case", ["register_staged_f32", "software_pipelined_f16"])
def test_grouped_call_in_graph(case):
    torch = _torch()
    if case == "register_staged_f32":
        dtype, req, shapes = "f32", None, [(256, 256, 256), (100, 130, 70), (64, 512, 33)]
    else:  # the persistent software-pipelined grouped kernel: aligned, whole k-tiles
        dtype, req, shapes = "f16", dg.request(schedule=5), [(512, 512, 256), (300, 264, 128), (257, 776, 512)]
    ops = [operands(torch, M, N, K, dtype, "N") for (M, N, K) in shapes]
    C = [[torch.zeros(M * N, dtype=torch.float32, device="cuda") for (M, N, K) in shapes] for _ in range(2)]
    print(f"graph case grouped {case}", flush=True)

    def probs(i):
        return [dg.problem(M, N, K, A.data_ptr(), lda, B.data_ptr(), ldb, C[i][j].data_ptr(), N)
                for j, ((M, N, K), (A, lda, B, ldb)) in enumerate(zip(shapes, ops))]

    def call(i, s):
        dg.gemm_grouped(0, 0, dg.DTYPE_CODE[dtype], probs(i), req, s)

    inputs = [t for (A, _, B, _) in ops for t in (A, B)]
    for i, t in enumerate(inputs):
        refill(torch, t, 100 + i)
    call(1, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with torch.cuda.graph(graph, stream=side):
        call(0, side.cuda_stream)
    for rep in range(3):
        for i, t in enumerate(inputs):
            refill(torch, t, 1000 * (rep + 1) + i)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        call(1, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for j in range(len(shapes)):
            assert torch.equal(C[0][j], C[1][j]), f"replay {rep}, problem {j} differs from the eager call"
