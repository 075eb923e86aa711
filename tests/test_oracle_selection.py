"""Pins for the active-row selection (CPU only): brute force by Python's sort."""
import itertools
import math

import numpy as np
import pytest

from oracle.selection import FORCE_EXCLUDED, FORCE_ON, select_thresh_cap, select_topk

NAN = float("nan")


def sort_reference(scores, force, k):
    """Independent definition: sort candidates with Python's stable sort on a tuple key."""
    cands = [i for i in range(len(scores)) if force[i] != FORCE_EXCLUDED]
    def key(i):
        s = scores[i]
        forced = force[i] == FORCE_ON
        isnan = math.isnan(s)
        return (0 if forced else 1, 1 if (not forced and isnan) else 0,
                0.0 if (forced or isnan) else -(s + 0.0), i)
    return sorted(sorted(cands, key=key)[:k])


VALUES = [1.0, 0.5, 0.5, -0.0, 0.0, NAN, float("inf"), float("-inf")]


@pytest.mark.parametrize("S", [1, 2, 3, 5, 8])
def test_exhaustive_small(S):
    rng = np.random.default_rng(S)
    for trial in range(300 if S > 3 else 60):
        scores = [VALUES[j] for j in rng.integers(0, len(VALUES), S)]
        force = rng.choice([0, 0, 0, 1, 2], S).astype(np.uint8)
        for k in range(0, S + 2):
            got = select_topk(np.array(scores), force, k).tolist()
            assert got == sort_reference(scores, force, k), (scores, force.tolist(), k)


def test_all_permutations_of_tied_values():
    base = [0.25, 0.25, 0.75, -0.0, 0.0, 0.75]
    for perm in itertools.permutations(base):
        for k in range(7):
            got = select_topk(np.array(perm), None, k).tolist()
            assert got == sort_reference(list(perm), [0] * 6, k)


def test_all_equal_scores_take_lowest_indices():
    for S in (1, 7, 64):
        for k in (0, 1, S // 2, S):
            assert select_topk(np.full(S, 0.3), None, k).tolist() == list(range(k))


def test_nan_ranks_below_minus_infinity():
    s = np.array([NAN, float("-inf"), NAN, 2.0])
    assert select_topk(s, None, 2).tolist() == [1, 3]
    assert select_topk(s, None, 3).tolist() == [0, 1, 3]


def test_signed_zero_ties_by_index():
    s = np.array([-0.0, 0.0, -0.0])
    assert select_topk(s, None, 1).tolist() == [0]
    assert select_topk(np.array([0.0, -0.0]), None, 1).tolist() == [0]


def test_forced_and_excluded():
    s = np.array([5.0, 1.0, 9.0, 3.0, float("inf")])
    f = np.array([0, 1, 2, 0, 0], dtype=np.uint8)
    # forced row 1 first, row 2 excluded, then +inf (row 4), then 5.0 (row 0)
    assert select_topk(s, f, 1).tolist() == [1]
    assert select_topk(s, f, 3).tolist() == [0, 1, 4]
    assert select_topk(s, f, 10).tolist() == [0, 1, 3, 4]


def test_thresh_cap():
    s = np.array([0.02, 0.001, 0.5, 0.011, 0.0, 0.3])
    f = np.array([0, 0, 0, 0, 1, 0], dtype=np.uint8)
    # strictly above tau = 0.01: rows 0, 2, 3, 5 plus forced row 4
    assert select_thresh_cap(s, f, 0.01, 10).tolist() == [0, 2, 3, 4, 5]
    # cap 3: forced first, then 0.5 and 0.3
    assert select_thresh_cap(s, f, 0.01, 3).tolist() == [2, 4, 5]
    assert select_thresh_cap(s, f, 0.02, 10).tolist() == [2, 4, 5]
    assert select_thresh_cap(s, None, 1.0, 10).tolist() == []
