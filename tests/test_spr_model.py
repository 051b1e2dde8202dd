"""CPU model of the register-staged software-pipelined kernel's chunk addressing.

The kernel (schedule 7) stages each lane's 16-byte chunks of the A and B tiles
global -> registers -> LDS. This model restates, in numpy, the kernel's formulas for
which chunk a lane owns, the address it loads from (a chunk that straddles K, or N for
a row-major B, is loaded as the 8 elements ending at the last valid one; a chunk past
the end is loaded from the row start; rows past M or N are clamped) and the shift that
puts the kept elements in place (keep_first8, as the kernel's 128-bit shift on two
64-bit halves). It checks, for ragged shapes, both B layouts and both wave counts,
that every load stays inside the row's valid elements and that the LDS tile built
from the loads equals the logical tile zero-padded past K and N.
"""
from __future__ import annotations

import numpy as np
import pytest

M64 = (1 << 64) - 1


def kmaj32_swz(r):
    return (r >> 2) & 3


def nmaj32_swz(k):
    return (k & 3) << 2


def keep_first8(w: np.ndarray, v: int) -> np.ndarray:
    """The kernel's keep_first8 on 8 uint16 values, through its 64-bit halves."""
    if v >= 8:
        return w.copy()
    if v <= 0:
        return np.zeros(8, dtype=np.uint16)
    u = [int(x) for x in w.view(np.uint32)]
    lo, hi = u[0] | (u[1] << 32), u[2] | (u[3] << 32)
    s = 16 * (8 - v)
    if s >= 64:
        olo, ohi = hi >> (s - 64), 0
    else:
        olo, ohi = ((lo >> s) | (hi << (64 - s))) & M64, hi >> s
    out = np.array([olo & 0xFFFFFFFF, olo >> 32, ohi & 0xFFFFFFFF, ohi >> 32], dtype=np.uint32)
    return out.view(np.uint16)


@pytest.mark.parametrize("v", range(-2, 11))
def test_keep_first8_is_a_shift_by_elements(v):
    w = np.arange(1, 9, dtype=np.uint16) * 0x1111
    got = keep_first8(w, v)
    want = np.zeros(8, dtype=np.uint16)
    for e in range(8):
        if e < min(v, 8):
            want[e] = w[e + 8 - min(v, 8)]
    assert np.array_equal(got, want)


def stage_tiles(M, N, K, lda, ldb, opb, nw, tm, tn, t, a_store, b_store):
    """The LDS A and B tiles (k-major A 256 x 32; B k-major 256 x 32 or n-major 32 x 256,
    in logical order after undoing the swizzle) of k-tile t of output tile (tm, tn),
    built the way the kernel's lanes load and write them; asserts every load is inside
    its row's valid range."""
    cpb = 16 // nw
    m0, n0 = 256 * tm, 256 * tn
    nk = -(-K // 32)
    tail = (K % 32 != 0) and t == nk - 1
    nedge = opb == 0 and n0 + 256 > N
    A_lds = np.full((256, 32), 0xFFFF, dtype=np.uint16)
    B_lds = np.full((256, 32) if opb == 1 else (32, 256), 0xFFFF, dtype=np.uint16)
    for wave in range(nw):
        for lane in range(64):
            for i in range(cpb):
                b = wave * cpb + i
                # A (and a column-major B): row b*16 + lane/4, logical chunk (lane&3)^swz
                row = b * 16 + (lane >> 2)
                kc = ((lane & 3) ^ kmaj32_swz(row)) << 3
                for which, store, ld, rows_valid in (("A", a_store, lda, M), ("B", b_store, ldb, N)):
                    if which == "B" and opb == 0:
                        continue
                    r = min((m0 if which == "A" else n0) + row, rows_valid - 1)
                    k0 = t * 32 + kc
                    start = k0
                    if tail:
                        vk = K - k0
                        if vk < 8:
                            start = K - 8 if vk > 0 else 0
                    assert 0 <= start and start + 8 <= K, (which, row, kc, start)
                    w = store[r * ld + start:r * ld + start + 8]
                    data = keep_first8(w, K - k0) if tail else w
                    (A_lds if which == "A" else B_lds)[row, kc:kc + 8] = data
                if opb == 0:
                    krow = b * 2 + (lane >> 5)
                    chunk = (lane & 31) ^ nmaj32_swz(krow)
                    col = n0 + chunk * 8
                    v = N - col
                    colr = col if v >= 8 else (N - 8 if v > 0 else 0)
                    nv = max(0, min(8, v))
                    k = t * 32 + krow
                    kr = k if not (tail and k >= K) else K - 1
                    assert 0 <= kr < K and 0 <= colr and colr + 8 <= N
                    w = b_store[kr * ldb + colr:kr * ldb + colr + 8]
                    data = keep_first8(w, nv) if nedge else w
                    if tail and k >= K:
                        data = np.zeros(8, dtype=np.uint16)
                    B_lds[krow, chunk * 8:chunk * 8 + 8] = data
    return A_lds, B_lds


@pytest.mark.parametrize("nw", [4, 8])
@pytest.mark.parametrize("opb", [0, 1])
@pytest.mark.parametrize("shape", [(300, 264, 37), (513, 777, 1037), (100, 9, 13), (257, 263, 71), (65, 65, 9),
                                   (40, 8, 8), (256, 256, 64)])
def test_staged_tiles_equal_zero_padded_operands(nw, opb, shape):
    M, N, K = shape
    if opb == 0 and N < 8:
        pytest.skip("row-major B needs N >= 8")
    rng = np.random.default_rng(M + N + K)
    lda = K + 3
    ldb = (N if opb == 0 else K) + 5
    a_store = rng.integers(1, 0xFFFF, M * lda, dtype=np.uint16)
    b_rows = K if opb == 0 else N
    b_store = rng.integers(1, 0xFFFF, b_rows * ldb, dtype=np.uint16)
    A = a_store.reshape(M, lda)[:, :K]
    Bl = b_store.reshape(b_rows, ldb)[:, :(N if opb == 0 else K)]
    nk = -(-K // 32)
    tiles = {(0, 0), (-(-M // 256) - 1, -(-N // 256) - 1)}
    for tm, tn in tiles:
        for t in sorted({0, nk - 1}):
            A_lds, B_lds = stage_tiles(M, N, K, lda, ldb, opb, nw, tm, tn, t, a_store, b_store)
            m0, n0, k0 = 256 * tm, 256 * tn, 32 * t
            kv = min(32, K - k0)
            rows = min(256, M - m0)
            # rows inside M: the logical A tile, zero past K
            assert np.array_equal(A_lds[:rows, :kv], A[m0:m0 + rows, k0:k0 + kv])
            assert np.all(A_lds[:rows, kv:] == 0)
            cols = min(256, N - n0)
            if opb == 1:
                assert np.array_equal(B_lds[:cols, :kv], Bl[n0:n0 + cols, k0:k0 + kv])
                assert np.all(B_lds[:cols, kv:] == 0)
            else:
                assert np.array_equal(B_lds[:kv, :cols], Bl[k0:k0 + kv, n0:n0 + cols])
                assert np.all(B_lds[kv:, :] == 0)
                assert np.all(B_lds[:kv, cols:] == 0)
            # every LDS position was written (the data never holds the 0xFFFF fill)
            assert not np.any(A_lds == 0xFFFF) and not np.any(B_lds == 0xFFFF)
