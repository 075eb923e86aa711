"""Dilated unmasking schedule (test infrastructure).

DUS, "Plan for Speed: Dilated Scheduling for Masked Diffusion Language
Models" (gist.science summary, technical summary section 2, algorithm
design): a block of B positions is split into non-adjacent dilated groups that
are unmasked coarse to fine in R = ceil(log_a B) rounds (a > 1, usually 2);
early rounds use a large stride, later rounds fill the gaps.  The lay section
illustrates it with positions 1, 5, 9, 13, 17, then 3, 7, 11, 15, then the
rest.

Reading: round r (0-based) uses stride a^(R-1-r) and takes every position
(0-based, within the block) that is a multiple of that stride and was not
taken by an earlier round.
"""
from __future__ import annotations


def n_rounds(block: int, a: int = 2) -> int:
    """Smallest R with a**R >= block (= ceil(log_a block)), computed exactly."""
    if block < 1 or a < 2:
        raise ValueError("block >= 1 and a >= 2 required")
    r, p = 0, 1
    while p < block:
        p *= a
        r += 1
    return r


def dus_rounds(block: int, a: int = 2, rounds: int | None = None) -> list[list[int]]:
    """Positions unmasked in each round, 0-based within the block."""
    R = n_rounds(block, a) if rounds is None else int(rounds)
    if R == 0:
        return [[0]] if block == 1 else []
    taken = [False] * block
    out = []
    for r in range(R):
        stride = a ** (R - 1 - r)
        grp = [p for p in range(0, block, stride) if not taken[p]]
        for p in grp:
            taken[p] = True
        out.append(grp)
    return out
