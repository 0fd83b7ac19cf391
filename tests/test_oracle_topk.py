"""Pins for the top-K oracle: a hand-ordered row and an O(n^2) rank count."""

import math

import numpy as np
import pytest

from oracle.topk import topk_row, topk_rows
from synth import topk_planted_rows


def rank_by_counting(row):
    """rank[j] = number of entries that must come before j (independent definition)."""
    n = len(row)
    rank = np.zeros(n, dtype=np.int64)
    for j in range(n):
        a = float(row[j])
        for i in range(n):
            if i == j:
                continue
            b = float(row[i])
            if math.isnan(a):
                before = math.isnan(b) and i < j or not math.isnan(b)
            elif math.isnan(b):
                before = False
            else:
                before = b > a or (b == a and i < j)
            rank[j] += before
    return rank


def test_hand_ordered_row():
    nan, inf = float("nan"), float("inf")
    row = np.array([1.0, nan, -inf, 0.0, -0.0, 1.0, 3.0, -0.0], dtype=np.float32)
    vals, ids = topk_row(row, 8)
    assert list(ids) == [6, 0, 5, 3, 4, 7, 2, 1]
    # bits are copied: -0 stays -0
    assert np.signbit(vals[4]) and not np.signbit(vals[3])
    assert math.isnan(vals[7])


def test_all_equal_row_takes_lowest_ids():
    vals, ids = topk_row(np.full(100, 2.5, dtype=np.float32), 10)
    assert list(ids) == list(range(10))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_matches_rank_counting(seed):
    rng = np.random.default_rng(seed)
    row = rng.integers(-3, 4, 60).astype(np.float32)  # many exact ties
    row[rng.choice(60, 4, replace=False)] = np.nan
    row[rng.choice(60, 3, replace=False)] = -np.inf
    row[rng.choice(60, 3, replace=False)] = -0.0
    rank = rank_by_counting(row)
    for K in (1, 7, 16, 60):
        _, ids = topk_row(row, K)
        assert list(ids) == list(np.argsort(rank)[:K])


def test_planted_rows_small():
    x = topk_planted_rows(5, rows=4, vocab=300, K=16)
    vals, ids = topk_rows(x, 16)
    for r in range(4):
        rank = rank_by_counting(x[r])
        assert list(ids[r]) == list(np.argsort(rank)[:16])
        assert np.array_equal(vals[r].view(np.uint32), x[r, ids[r]].view(np.uint32))
    # the row with fewer finite values than K ends in -inf then NaN
    assert np.isneginf(vals[2, 8]) and np.isfinite(vals[2, 7])
