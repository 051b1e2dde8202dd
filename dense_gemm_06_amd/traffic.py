"""Closed-form global-memory traffic of a block-tiled GEMM.

"Shared memory and tensor cores", section 13.1: a block computing a BM x BN tile
of C loads a BM x K panel of A and a K x BN panel of B once, so a square N^3
problem reads (N/BM)(N/BN)(BM + BN)K elements, against 2N^3 for the naive
kernel, and the intensity is BM*BN / (2(BM + BN)) FLOP per byte for 4-byte
elements (T/4 for a square T x T tile). The compulsory traffic reads each input
once and writes C once.

For ragged shapes the tiled count is the exact masked form
M*K*ceil(N/BN) + K*N*ceil(M/BM) elements: every A row is re-read once per
column of tiles and every B column once per row of tiles. Bytes are elements
times the input element size (4 for fp32, 2 for fp16/bf16).
"""
from __future__ import annotations

from math import ceil


def tiled_elements(M: int, N: int, K: int, BM: int, BN: int) -> int:
    """Input elements loaded by a BM x BN block tiling (no cache reuse between blocks)."""
    return M * K * ceil(N / BN) + K * N * ceil(M / BM)


def tiled_bytes(M: int, N: int, K: int, BM: int, BN: int, elem_size: int) -> int:
    return tiled_elements(M, N, K, BM, BN) * elem_size


def naive_elements(M: int, N: int, K: int) -> int:
    """One A and one B element per multiply-add."""
    return 2 * M * N * K


def compulsory_read_bytes(M: int, N: int, K: int, elem_size: int) -> int:
    return (M * K + K * N) * elem_size


def compulsory_bytes(M: int, N: int, K: int, elem_size: int, c_size: int = 4) -> int:
    """Read A and B once, write C once (C is fp32 for every input dtype here)."""
    return compulsory_read_bytes(M, N, K, elem_size) + M * N * c_size


def intensity(BM: int, BN: int, elem_size: int = 4) -> float:
    """FLOP per byte of tiled input traffic: 2*BM*BN*K FLOP over (BM+BN)*K*elem_size bytes."""
    return 2.0 * BM * BN / ((BM + BN) * elem_size)


def flops(M: int, N: int, K: int) -> int:
    return 2 * M * N * K


def table_13_1(N: int = 4096):
    """The chapter's N^3 fp32 table: rows of (scheme, bytes, FLOP per byte), then compulsory bytes."""
    f = flops(N, N, N)
    rows = [("naive: 2 loads per FMA", 4 * naive_elements(N, N, N))]
    for T in (16, 32, 64, 128):
        rows.append((f"block tile {T}x{T} in shared memory", 4 * tiled_elements(N, N, N, T, T)))
    return [(name, b, f / b) for name, b in rows], compulsory_read_bytes(N, N, N, 4)


def format_table_13_1(N: int = 4096) -> list[str]:
    """The table formatted as the chapter prints it (GB and FLOP/byte with one decimal)."""
    rows, comp = table_13_1(N)
    out = [f"N = {N}: {flops(N, N, N) / 1e9:.0f} GFLOP per GEMM"]
    out += [f"{name} | {b / 1e9:.1f} | {fpb:.1f}" for name, b, fpb in rows]
    out.append(f"compulsory (each input read once): {comp / 1e6:.0f} MB")
    return out
