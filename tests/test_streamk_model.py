"""CPU model of the stream-K schedule of the persistent software-pipelined kernel.

A restatement of the share bounds of dense_gemm_06_amd/csrc/streamk.h ("Shared
memory and tensor cores" section 13.10: the tail tiles' k-tiles dealt out as
equal, contiguous shares), checked for what the kernel and its fixup launch rely
on, over every tail size, k-tile count and share count in a range:

* the shares tile the iteration space: non-decreasing bounds from 0 to S * KT;
* every non-empty piece spans at least 4 k-tiles (the copy stream runs 3 ahead);
* a share meets at most two tiles (two workspace slots per workgroup);
* the fixup's walk over a tile (from the share that holds its first k-tile)
  visits exactly the pieces that lie in it, in k order, with the slot each piece
  was written to, and skips the tiles one piece covers (those go to C directly).

The planner's side (which requests it accepts) is exercised by plan_fuzz.cpp.
"""
from __future__ import annotations

import pytest

MIN_PIECE = 4


def bound(w, G, iters, KT):
    b = w * iters // G
    r = b % KT
    if r:
        if r < MIN_PIECE:
            b -= r
        elif KT - r < MIN_PIECE:
            b += KT - r
    return b


def piece(w, p, G, S, KT):
    iters = S * KT
    b0, b1 = bound(w, G, iters, KT), bound(w + 1, G, iters, KT)
    s = b0 if p == 0 else (b0 // KT + 1) * KT
    if s >= b1:
        return None
    t = s // KT
    e = min(b1, (t + 1) * KT)
    return t, s - t * KT, e - s


def owner(it, G, iters, KT):
    lo, hi = 0, G - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if bound(mid, G, iters, KT) <= it:
            lo = mid
        else:
            hi = mid - 1
    return lo


def fixup_walk(t, G, S, KT):
    """(w, slot) pairs the fixup adds for tail tile t, or None if one piece covers it."""
    iters = S * KT
    lo, hi = t * KT, (t + 1) * KT
    w0 = owner(lo, G, iters, KT)
    if bound(w0 + 1, G, iters, KT) >= hi:
        return None
    out = []
    for w in range(w0, G):
        b0, b1 = bound(w, G, iters, KT), bound(w + 1, G, iters, KT)
        if b0 >= hi:
            break
        if b1 <= b0 or b1 <= lo:
            continue
        out.append((w, 2 * w + (0 if b0 >= lo else 1)))
    return out


def schedules():
    # every tail size and share count for grids of up to 24, a sample for 256
    for KT in (8, 9, 13, 16, 31, 32, 64, 65):
        for G in (2, 3, 5, 8, 13, 24):
            for S in range(1, G):
                for width in range(S + 1, G + 1):
                    if (S * KT) // width >= MIN_PIECE:
                        yield KT, S, width
        for S in (1, 2, 33, 100, 255):
            for width in sorted({S + 1, 2 * S, 66, 129, 256}):
                if S < width <= 256 and (S * KT) // width >= MIN_PIECE:
                    yield KT, S, width


def test_streamk_schedule_invariants():
    n = 0
    for KT, S, G in schedules():
        iters = S * KT
        b = [bound(w, G, iters, KT) for w in range(G + 1)]
        assert b[0] == 0 and b[G] == iters
        assert all(b[i] <= b[i + 1] for i in range(G))
        # pieces per workgroup, and coverage of every (tile, k-tile) exactly once
        cover = {}
        written = {}
        for w in range(G):
            got = [piece(w, p, G, S, KT) for p in (0, 1)]
            for p in (0, 1):
                pc = got[p]
                if pc is None:
                    continue
                t, kb, nk = pc
                assert 0 <= t < S and nk >= MIN_PIECE and kb + nk <= KT, (KT, S, G, w, pc)
                for k in range(kb, kb + nk):
                    assert (t, k) not in cover
                    cover[(t, k)] = w
                if nk < KT:
                    written[(t, kb)] = (w, 2 * w + p)
            # the two pieces are the whole share (it meets at most two tiles)
            span = sum(pc[2] for pc in got if pc)
            assert span == b[w + 1] - b[w]
        assert len(cover) == iters
        # the fixup's walk: exactly the partial pieces of each split tile, in k order
        for t in range(S):
            walk = fixup_walk(t, G, S, KT)
            parts = sorted((kb, ws) for (tt, kb), ws in written.items() if tt == t)
            if walk is None:
                assert not parts, (KT, S, G, t)
            else:
                assert walk == [ws for _, ws in parts], (KT, S, G, t)
        n += 1
    assert n > 500


@pytest.mark.parametrize("KT,S,G", [(64, 33, 66), (16, 4, 5), (8, 8, 12)])
def test_streamk_examples(KT, S, G):
    """Hand-checked cases: 33 tiles of 64 k-tiles over 66 workgroups are halves of
    tiles; 4 tiles of 16 over 5 move the bound at 51 down to 48; 8 tiles of 8 over 12
    move bounds 5 and 10 both to 8, leaving one share empty."""
    iters = S * KT
    b = [bound(w, G, iters, KT) for w in range(G + 1)]
    if (KT, S, G) == (64, 33, 66):
        assert b == [32 * w for w in range(67)]
    elif (KT, S, G) == (16, 4, 5):
        assert b == [0, 12, 25, 38, 48, 64]
    else:
        assert b[:4] == [0, 8, 8, 16] and piece(1, 0, G, S, KT) is None
