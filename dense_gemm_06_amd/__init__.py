"""Python binding of the MI355X dense GEMM library (libdensegemm.so).

The functions mirror the C ABI in include/gemm.h one to one (gemm, gemm_ex,
gemm_ex_workspace, gemm_ex_noalloc, gemm_ex_epilogue, gemm_plan, gemm_plan_workspace, gemm_grouped, gemm_grouped_plan, gemm_strided_batched,
gemm_menu_size / gemm_menu_entry, gemm_device_info, gemm_status_string,
gemm_last_error) and only marshal arguments: every step of the product runs in
the library's HIP kernels. A nonzero status raises
GemmError carrying the library's own description.

``gemm_tensors`` is a convenience for torch tensors: it reads pointers, leading
dimensions and the current stream off the tensors and calls gemm_ex. Torch
provides device memory and streams only.

The library is loaded on first use. If it has not been built (``python -m
dense_gemm_06_amd.build``) every call raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, fields

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdensegemm.so")

GEMM_F32, GEMM_F16, GEMM_BF16 = 0, 1, 2
GEMM_OP_N, GEMM_OP_T = 0, 1
GEMM_OK = 0
GEMM_ERR_INVALID_VALUE = 1
GEMM_ERR_NULL_POINTER = 2
GEMM_ERR_UNSUPPORTED = 3
GEMM_ERR_DEVICE = 4
GEMM_ERR_LAUNCH = 5
GEMM_VARIANT_AUTO, GEMM_VARIANT_LDS, GEMM_VARIANT_MFMA = 0, 1, 2
GEMM_NOALLOC_SCRATCH_BYTES = 32 << 20   # the fixed scratch of gemm_ex_noalloc (include/gemm.h)

DTYPE_CODE = {"f32": GEMM_F32, "f16": GEMM_F16, "bf16": GEMM_BF16}
OP_CODE = {"N": GEMM_OP_N, "T": GEMM_OP_T}


class gemm_config(ctypes.Structure):
    _fields_ = [
        ("variant", ctypes.c_int32), ("bm", ctypes.c_int32), ("bn", ctypes.c_int32), ("bk", ctypes.c_int32),
        ("vec", ctypes.c_int32), ("xcd_remap", ctypes.c_int32), ("group_m", ctypes.c_int32),
        ("waves_m", ctypes.c_int32), ("waves_n", ctypes.c_int32),
        ("thread_m", ctypes.c_int32), ("thread_n", ctypes.c_int32),
        ("threads", ctypes.c_int32), ("lds_bytes", ctypes.c_int32), ("grid", ctypes.c_int32),
        ("kernel_id", ctypes.c_int32), ("schedule", ctypes.c_int32),
        ("tiles_m", ctypes.c_int64), ("tiles_n", ctypes.c_int64),
        ("est_cycles", ctypes.c_double),
        ("tiles_total", ctypes.c_int64), ("launches", ctypes.c_int32), ("max_grid", ctypes.c_int32),
        ("split_k", ctypes.c_int32), ("k_chunk", ctypes.c_int32), ("workspace_bytes", ctypes.c_int64),
        ("pack", ctypes.c_int32), ("stream_k", ctypes.c_int32), ("sk_width", ctypes.c_int32),
        ("reserved", ctypes.c_int32), ("reserved2", ctypes.c_int32),
    ]

    def as_dict(self) -> dict:
        return {f[0]: getattr(self, f[0]) for f in self._fields_}


def request(variant: int = GEMM_VARIANT_AUTO, bm: int = 0, bn: int = 0, vec: int = -1,
            xcd_remap: int = -1, group_m: int = 0, waves_m: int = 0, waves_n: int = 0,
            schedule: int = 0, max_grid: int = 0, split_k: int = 0, pack: int = 0, threads: int = 0,
            stream_k: int = 0, sk_width: int = 0) -> gemm_config:
    """A gemm_config with only the "in" fields set (0 / -1: heuristic decides)."""
    c = gemm_config()
    c.variant, c.bm, c.bn, c.vec, c.xcd_remap, c.group_m = variant, bm, bn, vec, xcd_remap, group_m
    c.waves_m, c.waves_n, c.schedule, c.max_grid, c.split_k = waves_m, waves_n, schedule, max_grid, split_k
    c.pack, c.threads, c.stream_k, c.sk_width = pack, threads, stream_k, sk_width
    return c


GEMM_ACT_NONE, GEMM_ACT_RELU, GEMM_ACT_GELU_TANH = 0, 1, 2
ACT_CODE = {"none": GEMM_ACT_NONE, "relu": GEMM_ACT_RELU, "gelu_tanh": GEMM_ACT_GELU_TANH}


class gemm_epilogue(ctypes.Structure):
    """C = act(alpha * (A @ B) + beta * R + bias), stored as out_dtype (see include/gemm.h)."""
    _fields_ = [
        ("alpha", ctypes.c_float), ("beta", ctypes.c_float), ("R", ctypes.c_void_p), ("ldr", ctypes.c_int64),
        ("bias", ctypes.c_void_p), ("activation", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
    ]


def epilogue(alpha=1.0, beta=0.0, R=None, ldr=0, bias=None, activation="none", out_dtype="f32") -> gemm_epilogue:
    e = gemm_epilogue()
    e.alpha, e.beta, e.R, e.ldr, e.bias = alpha, beta, R, ldr, bias
    e.activation = ACT_CODE[activation] if isinstance(activation, str) else activation
    e.out_dtype = DTYPE_CODE[out_dtype] if isinstance(out_dtype, str) else out_dtype
    return e


class gemm_problem(ctypes.Structure):
    """One entry of a grouped call: `batch` problems of one shape at element strides."""
    _fields_ = [
        ("M", ctypes.c_int64), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("A", ctypes.c_void_p), ("lda", ctypes.c_int64), ("stride_a", ctypes.c_int64),
        ("B", ctypes.c_void_p), ("ldb", ctypes.c_int64), ("stride_b", ctypes.c_int64),
        ("C", ctypes.c_void_p), ("ldc", ctypes.c_int64), ("stride_c", ctypes.c_int64),
        ("batch", ctypes.c_int64),
    ]


def problem(M, N, K, A, lda, B, ldb, C, ldc, batch=1, stride_a=0, stride_b=0, stride_c=0) -> gemm_problem:
    p = gemm_problem()
    p.M, p.N, p.K, p.A, p.lda, p.stride_a = M, N, K, A, lda, stride_a
    p.B, p.ldb, p.stride_b, p.C, p.ldc, p.stride_c, p.batch = B, ldb, stride_b, C, ldc, stride_c, batch
    return p


class GemmError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {gemm_status_string(status)} -- {detail}")


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m dense_gemm_06_amd.build` "
                           "(there is no fallback implementation)")
    # Device memory and streams come from torch, so the library must run on the
    # same HIP runtime instance: load torch's runtime first, which then also
    # satisfies the library's libamdhip64 dependency. Loading the library first
    # would bring in a second HIP/HSA runtime and neither would see the device.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    cfgp = ctypes.POINTER(gemm_config)
    lib.gemm.argtypes = [i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, vp]
    lib.gemm.restype = i32
    lib.gemm_ex.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, cfgp, vp]
    lib.gemm_ex.restype = i32
    lib.gemm_plan.argtypes = [i32, i32, i64, i64, i64, i64, i64, i64, i32, ctypes.c_size_t, ctypes.c_size_t,
                              ctypes.c_size_t, i32, ctypes.c_char_p, cfgp, cfgp]
    lib.gemm_plan.restype = i32
    lib.gemm_ex_workspace.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, cfgp, vp, i64, vp]
    lib.gemm_ex_workspace.restype = i32
    lib.gemm_ex_noalloc.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, cfgp, vp]
    lib.gemm_ex_noalloc.restype = i32
    epip = ctypes.POINTER(gemm_epilogue)
    lib.gemm_plan_workspace.argtypes = [i32, i32, i64, i64, i64, i64, i64, i64, i32, ctypes.c_size_t,
                                        ctypes.c_size_t, ctypes.c_size_t, i32, ctypes.c_char_p, i64, epip, cfgp,
                                        cfgp]
    lib.gemm_ex_epilogue.argtypes = [i32, i32, i64, i64, i64, vp, i64, vp, i64, vp, i64, i32, epip, cfgp, vp, i64,
                                     vp]
    lib.gemm_ex_epilogue.restype = i32
    lib.gemm_plan_workspace.restype = i32
    probp = ctypes.POINTER(gemm_problem)
    lib.gemm_grouped.argtypes = [i32, i32, i32, probp, i32, cfgp, vp]
    lib.gemm_grouped.restype = i32
    lib.gemm_grouped_plan.argtypes = [i32, i32, i32, probp, i32, i32, ctypes.c_char_p, cfgp, cfgp]
    lib.gemm_grouped_plan.restype = i32
    lib.gemm_strided_batched.argtypes = [i32, i32, i64, i64, i64, vp, i64, i64, vp, i64, i64, vp, i64, i64, i64,
                                         i32, cfgp, vp]
    lib.gemm_strided_batched.restype = i32
    lib.gemm_menu_size.argtypes = []
    lib.gemm_menu_size.restype = i32
    lib.gemm_menu_entry.argtypes = [i32, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32), cfgp]
    lib.gemm_menu_entry.restype = i32
    lib.gemm_device_info.argtypes = [i32, ctypes.POINTER(i32), ctypes.c_char_p, i32]
    lib.gemm_device_info.restype = i32
    lib.gemm_status_string.argtypes = [i32]
    lib.gemm_status_string.restype = ctypes.c_char_p
    lib.gemm_last_error.argtypes = []
    lib.gemm_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (loads it on first call)."""
    return _load()


def gemm_status_string(status: int) -> str:
    return _load().gemm_status_string(status).decode()


def gemm_last_error() -> str:
    return _load().gemm_last_error().decode()


def _check(st: int, where: str):
    if st != GEMM_OK:
        raise GemmError(st, where, gemm_last_error())


def gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream=None, check=True) -> int:
    """C ABI gemm: pointers are device addresses (ints), dtype a GEMM_* code."""
    st = _load().gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream)
    if check:
        _check(st, "gemm")
    return st


def gemm_ex(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype, cfg: gemm_config | None = None,
            stream=None, check=True) -> int:
    st = _load().gemm_ex(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype,
                         ctypes.byref(cfg) if cfg is not None else None, stream)
    if check:
        _check(st, "gemm_ex")
    return st


def gemm_ex_workspace(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype, cfg: gemm_config | None = None,
                      workspace=None, workspace_bytes=0, stream=None, check=True) -> int:
    """gemm_ex with a device workspace (split K when it pays; see include/gemm.h)."""
    st = _load().gemm_ex_workspace(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype,
                                   ctypes.byref(cfg) if cfg is not None else None, workspace, workspace_bytes, stream)
    if check:
        _check(st, "gemm_ex_workspace")
    return st


def gemm_ex_noalloc(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype, cfg: gemm_config | None = None,
                    stream=None, check=True) -> int:
    """gemm_ex_workspace on the library's fixed scratch array (no allocation; calls that
    overlap on one GPU race on it)."""
    st = _load().gemm_ex_noalloc(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype,
                                 ctypes.byref(cfg) if cfg is not None else None, stream)
    if check:
        _check(st, "gemm_ex_noalloc")
    return st


def gemm_ex_epilogue(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype, epi: gemm_epilogue | None = None,
                     cfg: gemm_config | None = None, workspace=None, workspace_bytes=0, stream=None,
                     check=True) -> int:
    """The product with a fused epilogue (C's element type is epi.out_dtype)."""
    st = _load().gemm_ex_epilogue(opA, opB, M, N, K, A, lda, B, ldb, C, ldc, dtype,
                                  ctypes.byref(epi) if epi is not None else None,
                                  ctypes.byref(cfg) if cfg is not None else None, workspace, workspace_bytes, stream)
    if check:
        _check(st, "gemm_ex_epilogue")
    return st


def gemm_plan_workspace(opA, opB, M, N, K, lda, ldb, ldc, dtype, a_addr=0, b_addr=0, c_addr=0, num_cus=256,
                        arch="gfx950", workspace_bytes=0, req: gemm_config | None = None, check=True,
                        epi: gemm_epilogue | None = None):
    """Host-only: the configuration gemm_ex_workspace (or gemm_ex_epilogue with `epi`) would launch.
    Returns (status, gemm_config)."""
    out = gemm_config()
    st = _load().gemm_plan_workspace(opA, opB, M, N, K, lda, ldb, ldc, dtype, a_addr, b_addr, c_addr, num_cus,
                                     arch.encode() if arch is not None else None, workspace_bytes,
                                     ctypes.byref(epi) if epi is not None else None,
                                     ctypes.byref(req) if req is not None else None, ctypes.byref(out))
    if check:
        _check(st, "gemm_plan_workspace")
    return st, out


def gemm_plan(opA, opB, M, N, K, lda, ldb, ldc, dtype, a_addr=0, b_addr=0, c_addr=0, num_cus=256,
              arch="gfx950", req: gemm_config | None = None, check=True):
    """Host-only: the configuration gemm_ex would launch. Returns (status, gemm_config)."""
    out = gemm_config()
    st = _load().gemm_plan(opA, opB, M, N, K, lda, ldb, ldc, dtype, a_addr, b_addr, c_addr, num_cus,
                           arch.encode() if arch is not None else None,
                           ctypes.byref(req) if req is not None else None, ctypes.byref(out))
    if check:
        _check(st, "gemm_plan")
    return st, out


def _problem_array(problems):
    if problems is None:
        return None, 0
    arr = (gemm_problem * max(len(problems), 1))(*problems)
    return arr, len(problems)


def gemm_grouped(opA, opB, dtype, problems, cfg: gemm_config | None = None, stream=None, check=True,
                 count: int | None = None) -> int:
    """All problems (a list of gemm_problem) in one persistent launch per 16 entries."""
    arr, n = _problem_array(problems)
    st = _load().gemm_grouped(opA, opB, dtype, arr, n if count is None else count,
                              ctypes.byref(cfg) if cfg is not None else None, stream)
    if check:
        _check(st, "gemm_grouped")
    return st


def gemm_grouped_plan(opA, opB, dtype, problems, num_cus=256, arch="gfx950", req: gemm_config | None = None,
                      check=True, count: int | None = None):
    """Host-only: the configuration gemm_grouped would use. Returns (status, gemm_config)."""
    arr, n = _problem_array(problems)
    out = gemm_config()
    st = _load().gemm_grouped_plan(opA, opB, dtype, arr, n if count is None else count, num_cus,
                                   arch.encode() if arch is not None else None,
                                   ctypes.byref(req) if req is not None else None, ctypes.byref(out))
    if check:
        _check(st, "gemm_grouped_plan")
    return st, out


def gemm_strided_batched(opA, opB, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c, batch, dtype,
                         cfg: gemm_config | None = None, stream=None, check=True) -> int:
    st = _load().gemm_strided_batched(opA, opB, M, N, K, A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c,
                                      batch, dtype, ctypes.byref(cfg) if cfg is not None else None, stream)
    if check:
        _check(st, "gemm_strided_batched")
    return st


def gemm_menu():
    """Every compiled kernel configuration as dicts (variant, dtype, opb, tile fields)."""
    lib = _load()
    out = []
    for i in range(lib.gemm_menu_size()):
        v, d, o = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
        c = gemm_config()
        _check(lib.gemm_menu_entry(i, ctypes.byref(v), ctypes.byref(d), ctypes.byref(o), ctypes.byref(c)),
               "gemm_menu_entry")
        e = c.as_dict()
        e.update(variant=v.value, dtype=d.value, opb=o.value)
        out.append(e)
    return out


def gemm_device_info(device: int = 0):
    """(compute-unit count, architecture name) of a HIP device."""
    n = ctypes.c_int()
    buf = ctypes.create_string_buffer(64)
    _check(_load().gemm_device_info(device, ctypes.byref(n), buf, 64), "gemm_device_info")
    return n.value, buf.value.decode()


# ----------------------------------------------------------------------------- torch convenience
def _torch_dtype_code(t):
    import torch
    m = {torch.float32: GEMM_F32, torch.float16: GEMM_F16, torch.bfloat16: GEMM_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def gemm_tensors(A, B, C, op_b: str = "N", cfg: gemm_config | None = None, stream=None):
    """C[:M,:N] = A @ B for torch CUDA tensors (row-major views with unit inner stride).

    A: (M, K). B: (K, N) for op_b 'N', or its column-major storage (N, K) for op_b 'T'.
    C: (M, N) float32. Leading dimensions are taken from the row strides.
    """
    import torch
    if A.dim() != 2 or B.dim() != 2 or C.dim() != 2:
        raise ValueError("A, B, C must be 2-D")
    if A.stride(1) != 1 or B.stride(1) != 1 or C.stride(1) != 1:
        raise ValueError("A, B, C need unit stride along their last dimension")
    if C.dtype != torch.float32 or A.dtype != B.dtype:
        raise TypeError("C must be float32 and A, B share one dtype")
    M, K = A.shape
    N = B.shape[1] if op_b == "N" else B.shape[0]
    if (B.shape[0] if op_b == "N" else B.shape[1]) != K or tuple(C.shape) != (M, N):
        raise ValueError(f"shape mismatch: A {tuple(A.shape)}, B {tuple(B.shape)} (op {op_b}), C {tuple(C.shape)}")
    s = stream if stream is not None else torch.cuda.current_stream(A.device).cuda_stream
    return gemm_ex(GEMM_OP_N, OP_CODE[op_b], M, N, K, A.data_ptr(), max(A.stride(0), 1), B.data_ptr(),
                   max(B.stride(0), 1), C.data_ptr(), max(C.stride(0), 1), _torch_dtype_code(A), cfg, s)
