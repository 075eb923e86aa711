"""Pins for the SureLock lock rule, confidence unmasking and the DUS schedule (CPU only)."""
import math
import os

import numpy as np
import pytest

from oracle.dus import dus_rounds, n_rounds
from oracle.post import surelock_update, unmask_forced, unmask_topn

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "dus_worked_example.txt")


def test_lock_clauses():
    force = np.array([0, 0, 0, 0, 2, 0], dtype=np.uint8)
    conf = np.array([0.95, 0.95, 0.9, 0.99, 0.1, 0.99])
    kl = np.array([1e-3, 2e-3, 1e-4, 0.0, 5.0, 1e-4])
    rows = np.array([0, 1, 2, 3, 4])                  # row 5 not recomputed this step
    out = surelock_update(force, rows, conf, kl, True, 1e-3, 0.9)
    # row 0: KL == eps locks (at or below); row 1: KL above eps; row 2: conf == 0.9 is not > 0.9;
    # row 3 locks; row 4 stays locked (monotone); row 5 untouched
    assert out.tolist() == [2, 0, 0, 2, 2, 0]
    assert surelock_update(force, rows, conf, kl, False, 1e-3, 0.9).tolist() == force.tolist()


def test_lock_is_monotone_over_random_sequences():
    rng = np.random.default_rng(5)
    force = np.zeros(40, dtype=np.uint8)
    for _ in range(30):
        rows = np.nonzero(force != 2)[0]
        new = surelock_update(force, rows, rng.uniform(size=40), rng.uniform(size=40) * 2e-3, True, 1e-3, 0.5)
        assert np.all(new[force == 2] == 2)
        force = new


def test_unmask_top_n():
    mask = 99
    tok = np.array([[5, mask, mask, mask, mask, 7, mask]])
    conf = np.array([[0.99, 0.2, 0.8, 0.8, 0.1, 0.95, 0.9]])
    arg = np.array([[1, 11, 12, 13, 14, 15, 16]])
    out = unmask_topn(tok, conf, arg, mask, 1, 6, 2)     # block [1, 6): masked 1..4
    # 0.8 ties between positions 2 and 3 -> both; position 6 is outside the block
    assert out.tolist() == [[5, mask, 12, 13, mask, 7, mask]]
    out3 = unmask_topn(tok, conf, arg, mask, 0, 7, 10)
    assert out3.tolist() == [[5, 11, 12, 13, 14, 7, 16]]


def test_dus_worked_example_from_page():
    rounds = []
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                rounds.append([int(v) - 1 for v in line.split()])       # 1-based on the page
    n = 1 + max(max(r) for r in rounds)
    assert dus_rounds(n, 2, rounds=len(rounds)) == rounds


@pytest.mark.parametrize("a", [2, 3, 4])
def test_dus_round_count_and_partition(a):
    for B in range(1, 70):
        R = n_rounds(B, a)
        assert a ** max(R - 1, 0) < B <= a ** R or B == 1
        if B > 1:
            assert R == math.ceil(math.log(B) / math.log(a) - 1e-12)
        rs = dus_rounds(B, a)
        flat = sorted(p for r in rs for p in r)
        assert flat == list(range(B))
        # every round but the last has no two adjacent positions
        for r in rs[:-1]:
            assert all(q - p > 1 for p, q in zip(r, r[1:]))


def test_dus_block16_rounds():
    assert dus_rounds(16, 2) == [[0, 8], [4, 12], [2, 6, 10, 14], [1, 3, 5, 7, 9, 11, 13, 15]]


def test_unmask_forced_marks_only():
    mask = 99
    tok = np.array([[5, mask, mask, mask, 8, mask, mask]])
    force = np.array([[2, 1, 0, 1, 1, 2, 1]], dtype=np.uint8)
    arg = np.array([[1, 11, 12, 13, 14, 15, 16]])
    out = unmask_forced(tok, force, arg, mask, 0, 6)
    # position 4 is not masked, 5 is excluded (2), 6 lies outside [0, 6)
    assert out.tolist() == [[5, 11, mask, 13, 8, mask, mask]]


def test_dus_rounds_unmask_every_position_once():
    """Driving unmask_forced with the dilated rounds fills a block exactly once per position."""
    mask, lo, B = 50, 3, 16
    tok = np.full((1, lo + B + 2), mask)
    tok[0, :lo] = 1
    arg = np.arange(tok.size).reshape(tok.shape) + 100
    seen = np.zeros(tok.shape[1], dtype=int)
    for r in dus_rounds(B, 2):
        force = np.zeros(tok.shape, dtype=np.uint8)
        force[0, [lo + p for p in r]] = 1
        new = unmask_forced(tok, force, arg, mask, lo, lo + B)
        changed = np.nonzero(new[0] != tok[0])[0]
        assert sorted(changed.tolist()) == sorted(lo + p for p in r)
        seen[changed] += 1
        tok = new
    assert seen[lo:lo + B].tolist() == [1] * B and seen.sum() == B
    assert tok[0, lo + B:].tolist() == [mask, mask]


def test_unmask_forced_agrees_with_top_n_on_its_picks():
    """Marking exactly the top-n confident masked positions makes both rules agree."""
    rng = np.random.default_rng(11)
    mask = 7
    tok = rng.integers(0, 7, size=(3, 40))
    tok[rng.uniform(size=tok.shape) < 0.6] = mask
    conf = rng.uniform(size=tok.shape)
    arg = rng.integers(0, 7, size=tok.shape)
    n = 5
    force = np.zeros(tok.shape, dtype=np.uint8)
    for b in range(3):
        cand = [i for i in range(4, 36) if tok[b, i] == mask]
        for i in sorted(cand, key=lambda i: -conf[b, i])[:n]:
            force[b, i] = 1
    assert np.array_equal(unmask_forced(tok, force, arg, mask, 4, 36), unmask_topn(tok, conf, arg, mask, 4, 36, n))
