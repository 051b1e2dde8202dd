"""Helpers for the GPU tests: move seeded operands to the device and run the C ABI.

Torch is used for device memory and streams only; the product itself runs in the
library's kernels through dense_gemm_06_amd.gemm_ex.
"""
from __future__ import annotations

import numpy as np

import dense_gemm_06_amd as dg
import gemm_inputs as gi

SENTINEL = np.float32(-7.75e30)   # fills C padding and extra rows; must survive every call


def _torch():
    import torch
    return torch


def device_storage(arr: np.ndarray, offset_elems: int = 0):
    """Copy a flat storage array to the GPU; return (tensor, device address of element 0).

    offset_elems > 0 places the data that many elements past the start of the
    allocation, to produce base addresses that are not 16-byte aligned.
    """
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        host = torch.from_numpy(a.view(np.int16).copy())
    else:
        host = torch.from_numpy(a.copy())
    t = torch.empty(host.numel() + offset_elems + 8, dtype=host.dtype, device="cuda")
    t[offset_elems:offset_elems + host.numel()].copy_(host)
    return t, t.data_ptr() + offset_elems * t.element_size()


def run_ops(ops: gi.Operands, cfg=None, ldc: int | None = None, extra_rows: int = 2, a_off: int = 0,
            b_off: int = 0, c_off: int = 0, stream=None, fill=SENTINEL):
    """Run C = A @ B on the GPU for `ops`; return the whole C storage (rows x ldc) as float32.

    C is allocated with `extra_rows` rows beyond M and prefilled with `fill`, so
    writes outside C[:M, :N] are visible.
    """
    torch = _torch()
    ldc = ldc or max(1, ops.N)
    rows = ops.M + extra_rows
    At, a_ptr = device_storage(ops.A, a_off)
    Bt, b_ptr = device_storage(ops.B, b_off)
    Ct = torch.full((rows * ldc + c_off + 8,), float(fill), dtype=torch.float32, device="cuda")
    c_ptr = Ct.data_ptr() + c_off * 4
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    dg.gemm_ex(dg.GEMM_OP_N, dg.OP_CODE[ops.op_b], ops.M, ops.N, ops.K, a_ptr, ops.lda, b_ptr, ops.ldb,
               c_ptr, ldc, dg.DTYPE_CODE[ops.dtype], cfg, s)
    torch.cuda.synchronize()
    out = Ct[c_off:c_off + rows * ldc].cpu().numpy().reshape(rows, ldc)
    del At, Bt, Ct
    return out


def check_untouched(Cfull: np.ndarray, M: int, N: int, fill=SENTINEL):
    """Everything outside C[:M, :N] must still hold the fill value."""
    pad = Cfull[:M, N:]
    below = Cfull[M:, :]
    assert np.all(pad == fill), "kernel wrote into the ldc padding"
    assert np.all(below == fill), "kernel wrote rows at or beyond M"
