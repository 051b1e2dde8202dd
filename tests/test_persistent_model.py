"""CPU models of the persistent software-pipelined kernel (schedule 5 on a grid below
the tile count): the tile each workgroup takes per round, and the order of its LDS
copies, memory waits, barriers and fragment reads.

Tile order: the kernel's round_tile restated in Python; every tile must be taken by
exactly one (workgroup, round), rounds must be taken in order, each XCD's share of
a round must be a contiguous run, the runs must differ in length by at most one,
and a full round must match the one-tile-per-workgroup renumbering (XCD x gets tiles
x*G/8 .. x*G/8 + G/8 - 1).

Schedule: one wave's program order of the persistent loop, as issued copies (each
of CPB loads), waits on the vector-memory counter (loads and stores counted
together, completing in issue order for the purpose of this check), barriers,
fragment reads and the epilogue's use of one stage. The model asserts that a k-tile
is read only after every wave's copies of it completed before a barrier, that no
copy targets a stage read in the same barrier interval or the stage the epilogue
uses, and that a stage still holds the k-tile being read.
"""
from __future__ import annotations

import pytest

D = 3  # copy distance in k-tiles (4 stages)


def round_tile(bid, G, r, total, remap):
    base = r * G
    R = min(G, total - base)
    if not remap or G % 8:
        return base + bid if bid < R else -1
    x, local = bid & 7, bid >> 3
    q, rem = R >> 3, R & 7
    return base + x * q + min(x, rem) + local if local < q + (1 if x < rem else 0) else -1


@pytest.mark.parametrize("G", [1, 3, 8, 16, 23, 64, 192, 256])
@pytest.mark.parametrize("total", [1, 7, 24, 255, 256, 257, 576, 1024, 1031])
def test_round_tile_covers_each_tile_once(G, total):
    if G > total:
        pytest.skip("the planner caps the grid at the tile count")
    for remap in (0, 1):
        seen = {}
        for bid in range(G):
            r, prev = 0, None
            t = round_tile(bid, G, 0, total, remap)
            assert t >= 0, "every workgroup has a tile in round 0"
            while t >= 0:
                assert t not in seen and 0 <= t < total
                assert prev is None or t > prev
                seen[t] = (bid, r)
                r += 1
                prev = t
                t = round_tile(bid, G, r, total, remap)
            # once a round has no tile for the workgroup, no later round has one
            assert all(round_tile(bid, G, rr, total, remap) == -1 for rr in range(r, r + 3))
        assert sorted(seen) == list(range(total))
        if remap and G % 8 == 0:
            rounds = -(-total // G)
            for r in range(rounds):
                runs = {}
                for bid in range(G):
                    t = round_tile(bid, G, r, total, remap)
                    if t >= 0:
                        runs.setdefault(bid & 7, []).append(t)
                lens = [len(runs.get(x, [])) for x in range(8)]
                assert max(lens) - min(lens) <= 1
                for x, ts in runs.items():
                    assert ts == list(range(min(ts), min(ts) + len(ts))), "an XCD's run is contiguous"
                if total - r * G >= G:  # full round: the one-tile-per-workgroup renumbering
                    for bid in range(G):
                        assert round_tile(bid, G, r, total, remap) == r * G + (bid & 7) * (G >> 3) + (bid >> 3)


def run_schedule(nk, ntiles, cpb, mutation=None):
    q = []               # outstanding vector-memory operations in issue order
    done = {}            # (tile, k, half) -> stage, for completed copies
    visible = {}         # (tile, k) -> stage, published by a barrier
    last_into = {}       # stage -> what was last copied (or written) into it
    read_phase = set()   # stages read since the last barrier
    epi_stages = set()

    def copy(tile, k, half, st):
        assert st not in read_phase, ("copy into a stage read in this barrier interval", tile, k, st)
        assert st not in epi_stages, ("copy into the epilogue's stage", tile, k, st)
        q.extend([("copy", tile, k, half, st)] * cpb)
        last_into[st] = (tile, k)

    def wait(n):
        while len(q) > n:
            op = q.pop(0)
            if op[0] == "copy":
                done[op[1:4]] = op[4]

    def barrier():
        read_phase.clear()
        for (t, k, h), st in done.items():
            if (t, k, 1 - h) in done:
                visible[(t, k)] = st

    def read(tile, k, st):
        assert visible.get((tile, k)) == st, ("read before the copies completed", tile, k, st)
        assert last_into.get(st) == (tile, k), ("stage overwritten", tile, k, st, last_into.get(st))
        read_phase.add(st)

    sb, primed = 0, False
    for tile in range(ntiles):
        has_next = tile + 1 < ntiles
        if not primed:
            for t in range(D):
                copy(tile, t, 0, (sb + t) & 3)
                copy(tile, t, 1, (sb + t) & 3)
            wait(2 * cpb * (D - 1))
            barrier()
        read(tile, 0, sb & 3)
        for t in range(nk):
            last = t + D >= nk
            st, cst = (sb + t) & 3, (sb + t + D) & 3
            do_copy = not last or has_next
            ct, ck = (tile + 1, t + D - nk) if last else (tile, t + D)
            read(tile, t, st)                      # step (t, 0) reads step (t, 1)
            if do_copy:
                copy(ct, ck, 0, cst)
            if not (primed and t < (3 if mutation == "skip_three" else 2)):
                slack = cpb if mutation == "wait_slack" else 0
                wait(2 * cpb * (D - 2) + cpb + slack if do_copy else 2 * cpb * max(0, nk - t - 2) + slack)
            barrier()
            if t + 1 < nk:
                read(tile, t + 1, (st + 1) & 3)    # step (t, 1) reads step (t + 1, 0)
            if do_copy:
                copy(ct, ck, 1, cst)
        barrier()
        es = (sb + nk - (0 if mutation == "epilogue_stage" else 1)) & 3
        assert not any(op[0] == "copy" and op[4] == es for op in q), "copy in flight into the epilogue's stage"
        epi_stages.add(es)
        last_into[es] = ("epilogue",)
        if mutation != "no_final_wait":
            wait(0)                                # before the first store
        else:
            # stores issued with copies in flight may complete first: the counter
            # then says nothing about the copies, which the model shows by dropping
            # them from the count
            q[:] = [op for op in q if op[0] != "copy"]
        q.extend([("store",)] * 8)
        if not has_next:
            break
        barrier()
        epi_stages.clear()
        primed, sb = True, (sb + nk) & 3
    wait(0)


@pytest.mark.parametrize("nk", [4, 5, 6, 7, 8, 9, 33])
@pytest.mark.parametrize("ntiles", [1, 2, 3, 5])
@pytest.mark.parametrize("cpb", [1, 2])
def test_persistent_schedule_orders_copies_reads_and_epilogue(nk, ntiles, cpb):
    run_schedule(nk, ntiles, cpb)


@pytest.mark.parametrize("mutation", ["wait_slack", "skip_three", "epilogue_stage", "no_final_wait"])
def test_model_catches_plausible_slips(mutation):
    """Each plausible slip in the schedule makes the model fail, so that it is not
    vacuous: waiting for one copy too few, skipping the wait in a primed tile's
    first three iterations instead of two, running the epilogue through the stage of
    the next tile's first k-tile, and leaving the next tile's copies in flight at
    the epilogue's first store."""
    with pytest.raises(AssertionError):
        for nk in (4, 5, 8):
            for cpb in (1, 2):
                run_schedule(nk, 3, cpb, mutation=mutation)
