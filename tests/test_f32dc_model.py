"""CPU model of the fp32 direct-copy kernel (schedule 8, 64 x 64 tiles, two K groups,
four LDS stages): copy addresses, LDS layout and the order of copies, waits,
barriers and fragment reads.

Layout: the kernel's copy formulas restated in numpy (wave w copies blocks 2w, 2w+1
of A and of B; lane L of a block lands at byte 16 L and loads the logical chunk that
belongs there, rows past M or N clamped, row-major B chunks past N from column 0).
For ragged shapes and both B layouts every load must stay inside the matrix, and the
fragments read back with the kernel's read formulas must equal the logical tile
wherever they reach a stored row or column of C.

Schedule: the kernel's loop replayed as one wave's program order; every k-tile must
be complete before its fragments are read, no copy may land in a stage read since
the last barrier, and planted slips must fail the replay.
"""
from __future__ import annotations

import numpy as np
import pytest

BM = BN = 64
BK = 32


def copies(M, N, K, lda, ldb, opb, tm, tn, kg, kt_local, KG=2):
    """LDS contents (floats) of one group's stage for its local k-tile kt_local, built
    from the copies, and the (row, col) source index of every copied element."""
    m0, n0 = tm * BM, tn * BN
    k0 = (kt_local * KG + kg) * BK
    sA = np.full(BM * BK, np.nan)
    sB = np.full(BK * BN, np.nan)
    src = []
    for wave in range(4):
        for i in range(2):
            b = 2 * wave + i
            for L in range(64):
                row = b * 8 + (L >> 3)
                c = (L & 7) ^ (row & 7)
                r = min(m0 + row, M - 1)
                src.append(("A", r, k0 + 4 * c))
                sA[b * 256 + L * 4: b * 256 + L * 4 + 4] = [r * lda + k0 + 4 * c + e for e in range(4)]
                if opb == 1:
                    rn = min(n0 + row, N - 1)
                    src.append(("B", rn, k0 + 4 * c))
                    sB[b * 256 + L * 4: b * 256 + L * 4 + 4] = [rn * ldb + k0 + 4 * c + e for e in range(4)]
                else:
                    krow = b * 4 + (L >> 4)
                    col = n0 + 4 * (L & 15)
                    col = col if col < N else 0
                    src.append(("B", k0 + krow, col))
                    sB[b * 256 + L * 4: b * 256 + L * 4 + 4] = [(k0 + krow) * ldb + col + e for e in range(4)]
    return sA, sB, src


@pytest.mark.parametrize("opb", [0, 1])
@pytest.mark.parametrize("shape", [(64, 64, 64), (100, 68, 128), (1024, 1024, 1024), (65, 4, 64), (200, 1000, 192)])
def test_copies_in_bounds_and_fragments_equal_tile(opb, shape):
    M, N, K = shape
    lda = K + 4
    ldb = (N if opb == 0 else K) + 8
    tiles_m, tiles_n = -(-M // BM), -(-N // BN)
    for tm, tn in {(0, 0), (tiles_m - 1, tiles_n - 1)}:
        for kg in range(2):
            for ktl in {0, K // 64 - 1}:
                sA, sB, src = copies(M, N, K, lda, ldb, opb, tm, tn, kg, ktl)
                for which, r, c in src:
                    if which == "A":
                        assert 0 <= r < M and 0 <= c and c + 4 <= K
                    elif opb == 1:
                        assert 0 <= r < N and 0 <= c and c + 4 <= K
                    else:
                        assert 0 <= r < K and 0 <= c and c + 4 <= N
                m0, n0, k0 = tm * BM, tn * BN, (ktl * 2 + kg) * BK
                # fragment reads (both halves): A row ra, float4 at chunk (kk/4 + lg) ^ (ra & 7)
                for wave in range(4):
                    for lane in range(64):
                        l16, lg = lane & 15, lane >> 4
                        ra = wave * 16 + l16
                        for kk in (0, 16):
                            pos = (((kk >> 2) + lg) ^ (ra & 7)) << 2
                            got = sA[ra * BK + pos: ra * BK + pos + 4]
                            if m0 + ra < M:
                                want = [(m0 + ra) * lda + k0 + kk + 4 * lg + e for e in range(4)]
                                assert list(got) == want
                            for s in range(4):
                                if opb == 0:
                                    off = (kk + 4 * lg + s) * BN + 4 * l16
                                    got = sB[off: off + 4]
                                    for e in range(4):
                                        n = n0 + 4 * l16 + e
                                        if n < N:
                                            assert got[e] == (k0 + kk + 4 * lg + s) * ldb + n
                                else:
                                    r = s * 16 + l16
                                    pos = (((kk >> 2) + lg) ^ (r & 7)) << 2
                                    got = sB[r * BK + pos: r * BK + pos + 4]
                                    if n0 + r < N:
                                        assert list(got) == [(n0 + r) * ldb + k0 + kk + 4 * lg + e for e in range(4)]


def replay(nl, S=4, mutation=None):
    q, done, visible, last_into, read_phase = [], {}, {}, {}, set()

    def issue(t, st):
        assert st not in read_phase, ("copy into a stage read since the last barrier", t, st)
        q.extend([(t, st)] * 4)
        last_into[st] = t

    def wait(n):
        while len(q) > n:
            t, st = q.pop(0)
            done[t] = done.get(t, 0) + 1

    def barrier():
        read_phase.clear()
        for t, cnt in done.items():
            if cnt == 4:
                visible[t] = True

    def read(t, st):
        if t >= nl:
            read_phase.add(st)
            return
        assert visible.get(t) and last_into.get(st) == t, ("read before complete or after overwrite", t, st)
        read_phase.add(st)

    for t in range(min(S - 1, nl)):
        issue(t, t)
    wait(4 * max(0, min(S - 2, nl - 1) - 1) + (4 if mutation == "prologue" else 0))
    barrier()
    if nl > 0:
        read(0, 0)
    for lt in range(nl):
        st, nst = lt % S, (lt + 1) % S
        if lt + S - 1 < nl:
            issue(lt + S - 1, (lt + S - 1) % S if mutation != "stage" else nst)
        read(lt, st)
        read(lt + 1, nst)
        slack = 4 if mutation == "slack" else 0
        wait(4 * max(0, min(lt + S - 1, nl - 1) - (lt + 2)) + slack)
        barrier()
    wait(0)


@pytest.mark.parametrize("nl", [1, 2, 3, 4, 5, 8, 16])
def test_schedule_order(nl):
    replay(nl)


@pytest.mark.parametrize("mutation", ["prologue", "slack", "stage"])
def test_schedule_model_catches_slips(mutation):
    with pytest.raises(AssertionError):
        for nl in (2, 3, 4, 8):
            replay(nl, mutation=mutation)
