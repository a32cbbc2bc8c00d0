"""Pins the oracle's top-k selection to exhaustive search on tiny inputs and to its special cases.

Rule: candidates are complete regions 0..c-1; the current region c is always selected (within the k);
rank by score descending, lower region index first; output ascending, min(k, c+1) regions.
"""
import itertools

import numpy as np


def _brute(scores, c, k):
    """Subset of {0..c-1} of size min(k-1, c) with the largest score sum; among equal sums the
    lexicographically smallest ascending list (= lower indices win ties). Scores are integers so the
    sums are exact."""
    m = min(k - 1, c)
    best, best_sum = None, None
    for comb in itertools.combinations(range(c), m):
        s = sum(int(scores[i]) for i in comb)
        if best_sum is None or s > best_sum or (s == best_sum and list(comb) < list(best)):
            best, best_sum = comb, s
    return sorted(list(best) + [c])


def test_matches_exhaustive_search(oracle_lib):
    o = oracle_lib
    rng = np.random.default_rng(5)
    for trial in range(300):
        c = int(rng.integers(0, 12))
        k = int(rng.integers(1, 5))
        scores = rng.integers(0, 4, size=max(c, 1)).astype(np.float64)  # many ties
        got = o.select(scores, c, k).tolist()
        assert got == _brute(scores, c, k), (scores[:c], c, k, got)


def test_everything_selected_when_k_covers_all(oracle_lib):
    o = oracle_lib
    s = np.random.default_rng(1).uniform(size=50)
    assert o.select(s, 50, 512).tolist() == list(range(51))
    assert o.select(s, 10, 11).tolist() == list(range(11))


def test_all_zero_scores_take_lowest_indices(oracle_lib):
    o = oracle_lib
    s = np.zeros(1000)
    assert o.select(s, 1000, 512).tolist() == list(range(511)) + [1000]


def test_forced_region_even_with_lowest_score(oracle_lib):
    o = oracle_lib
    s = np.arange(600, 0, -1).astype(np.float64)  # region 599 lowest
    sel = o.select(s, 599, 512)
    assert 599 in sel.tolist() and len(sel) == 512
    assert sel.tolist() == list(range(511)) + [599]


def test_budget_never_exceeds_4096_tokens(oracle_lib):
    o = oracle_lib
    s = np.random.default_rng(2).uniform(size=5000)
    sel = o.select(s, 5000, 512)
    assert len(sel) == 512 and 8 * len(sel) <= 4096
    assert np.all(np.diff(sel) > 0)
