"""Bank-conflict model for LDS (shared-memory) access patterns.

"Shared memory and tensor cores", section 13.6: shared memory is split into
banks of 4-byte words, word w in bank w mod (number of banks); lanes reading the
same word share one broadcast, distinct words in one bank are served one per
pass, so an access takes as many passes as the most-loaded bank has distinct
words. The chapter models a 32-lane warp and 32 banks.

On gfx950 a wave has 64 lanes and the LDS serves a wave's access in several
phases of lanes. `passes` therefore takes the bank count and the number of
lanes served together in one phase as parameters; an access made of several
4-byte words per lane (ds_read_b64 / b128) is modelled word by word. The LDS
kernels' layouts are checked with this model in the tests before any run on
hardware; hardware bank-conflict counters remain the final word.
"""
from __future__ import annotations

from typing import Callable, Iterable


def passes(word_of_lane: Callable[[int], int | Iterable[int]], lanes: int = 32, banks: int = 32) -> int:
    """Worst-case passes for one access by `lanes` lanes over `banks` 4-byte banks."""
    words = set()
    for t in range(lanes):
        w = word_of_lane(t)
        if isinstance(w, int):
            words.add(w)
        else:
            words.update(w)
    per_bank: dict[int, set[int]] = {}
    for w in words:
        per_bank.setdefault(w % banks, set()).add(w)
    return max(len(s) for s in per_bank.values())


def wave_passes(word_of_lane: Callable[[int], int | Iterable[int]], wave: int = 64,
                phase_lanes: int = 32, banks: int = 32) -> int:
    """Sum of per-phase passes when a wave is served `phase_lanes` lanes at a time."""
    total = 0
    for p in range(0, wave, phase_lanes):
        total += passes(lambda t, p=p: word_of_lane(p + t), lanes=phase_lanes, banks=banks)
    return total
