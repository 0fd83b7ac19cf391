"""Pins for the sampler policy and the inverse-CDF draw.

The pages print no numbers for the policy, so these are constructed closed
forms: the textbook softmax (scipy) when every filter is off, one-hot cases,
and hand-worked 4-token distributions that fix the stage order.
"""

import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle.policy import draw, draw_weights, policy_row


def logits_for(probs, T):
    """Logits whose temperature-T softmax is exactly proportional to probs (up to exp rounding)."""
    return np.array([T * math.log(p) for p in probs], dtype=np.float64).astype(np.float32)


def test_temperature_zero_is_argmax_lowest_id():
    vals = np.array([1.0, 3.0, 3.0, 2.0], dtype=np.float32)
    ids = np.array([9, 7, 4, 1], dtype=np.int32)
    out_ids, probs = policy_row(vals, ids, 0.0, 20, 0.9, 0.1)
    assert list(out_ids) == [4] and list(probs) == [1.0]


@pytest.mark.parametrize("T", [0.7, 1.0, 2.5])
def test_filters_off_is_textbook_softmax(T):
    rng = np.random.default_rng(4)
    vals = (rng.standard_normal(64) * 3).astype(np.float32)
    ids = rng.permutation(1000)[:64].astype(np.int32)
    out_ids, probs = policy_row(vals, ids, T, 0, 1.0, 0.0)
    ref = softmax(vals.astype(np.float64) / np.float64(np.float32(T)))
    order = np.lexsort((ids, -vals))
    assert list(out_ids) == list(ids[order])
    np.testing.assert_allclose(probs.astype(np.float64), ref[order], rtol=2e-7, atol=1e-30)


def test_top_k_absent_is_20_and_zero_is_pool():
    vals = np.linspace(1.0, 0.0, 64, dtype=np.float32)
    ids = np.arange(64, dtype=np.int32)
    assert len(policy_row(vals, ids, 5.0, -1, 1.0, 0.0)[0]) == 20
    assert len(policy_row(vals, ids, 5.0, 0, 1.0, 0.0)[0]) == 64
    assert len(policy_row(vals, ids, 5.0, 1000, 1.0, 0.0)[0]) == 64
    assert len(policy_row(vals, ids, 5.0, 7, 1.0, 0.0)[0]) == 7
    o, p = policy_row(vals, ids, 5.0, 1, 1.0, 0.0)
    assert list(o) == [0] and list(p) == [1.0]


def test_min_p_hand_case():
    T = 1.0
    vals = logits_for([0.5, 0.3, 0.15, 0.05], T)
    ids = np.array([10, 11, 12, 13], dtype=np.int32)
    out_ids, probs = policy_row(vals, ids, T, 0, 1.0, 0.2)  # keep p >= 0.1
    assert list(out_ids) == [10, 11, 12]
    np.testing.assert_allclose(probs, np.array([0.5, 0.3, 0.15]) / 0.95, rtol=1e-6)


def test_top_p_keeps_the_crossing_candidate():
    T = 1.0
    vals = logits_for([0.5, 0.3, 0.15, 0.05], T)
    ids = np.array([10, 11, 12, 13], dtype=np.int32)
    out_ids, probs = policy_row(vals, ids, T, 0, 0.7, 0.0)  # mass before: 0, .5, .8
    assert list(out_ids) == [10, 11]
    np.testing.assert_allclose(probs, [0.625, 0.375], rtol=1e-6)
    out_ids, _ = policy_row(vals, ids, T, 0, 0.4, 0.0)
    assert list(out_ids) == [10]
    out_ids, _ = policy_row(vals, ids, T, 0, 0.0, 0.0)
    assert list(out_ids) == [10]


def test_min_p_runs_before_top_p():
    # min-p 0.3 leaves (.4,.3,.2)/.9; top-p .75 then keeps two (mass before: 0, .444, .778).
    # Top-p first would keep three (mass before: 0, .4, .7).
    T = 1.0
    vals = logits_for([0.4, 0.3, 0.2, 0.1], T)
    ids = np.array([1, 2, 3, 4], dtype=np.int32)
    out_ids, probs = policy_row(vals, ids, T, 0, 0.75, 0.3)
    assert list(out_ids) == [1, 2]
    np.testing.assert_allclose(probs, [4 / 7, 3 / 7], rtol=1e-6)


def test_top_k_runs_before_min_p():
    # top-k 2 leaves (.4,.3)/.7; min-p .8 needs p >= .8*.571 = .457 -> only the first.
    vals = logits_for([0.4, 0.3, 0.2, 0.1], 1.0)
    ids = np.array([1, 2, 3, 4], dtype=np.int32)
    assert list(policy_row(vals, ids, 1.0, 2, 1.0, 0.8)[0]) == [1]
    assert list(policy_row(vals, ids, 1.0, 2, 1.0, 0.7)[0]) == [1, 2]


def test_unsorted_candidates_and_specials():
    nan, inf = float("nan"), float("inf")
    vals = np.array([0.0, nan, 2.0, -inf, 2.0], dtype=np.float32)
    ids = np.array([5, 6, 9, 8, 3], dtype=np.int32)
    out_ids, probs = policy_row(vals, ids, 1.0, 0, 1.0, 0.0)
    assert list(out_ids) == [3, 9, 5]          # -inf and NaN carry no mass
    e = math.exp(-2.0)
    np.testing.assert_allclose(probs, np.array([1, 1, e]) / (2 + e), rtol=1e-7)
    # +inf logits share all the mass
    vals2 = np.array([inf, 1.0, inf], dtype=np.float32)
    out_ids, probs = policy_row(vals2, np.array([4, 5, 2], dtype=np.int32), 0.7, 0, 1.0, 0.0)
    assert list(out_ids) == [2, 4] and list(probs) == [0.5, 0.5]


def test_draw_inverse_cdf():
    p = np.array([0.25, 0.5, 0.25], dtype=np.float32)
    assert draw(p, 0.0) == 0
    assert draw(p, np.float32(0.25) - np.float32(2**-24)) == 0
    assert draw(p, 0.25) == 1
    assert draw(p, 0.75) == 2
    assert draw(p, 1 - 2**-24) == 2
    # zero-weight entries are never drawn
    assert draw_weights([0.0, 1.0, 0.0, 1.0], 0.0) == 1
    assert draw_weights([0.0, 1.0, 0.0, 1.0], 0.5) == 3


def test_draw_matches_probabilities_on_a_grid():
    p = np.array([0.125, 0.5, 0.25, 0.125], dtype=np.float32)
    grid = np.arange(1024, dtype=np.float64) / 1024
    counts = np.bincount([draw(p, u) for u in grid], minlength=4)
    assert list(counts) == [128, 512, 256, 128]
