"""Pins for the depth chooser and the window-cost model (oracle/depth.py).

* the break-even table printed in section 05 of "Speculative decoding on
  RDNA", recomputed from the page's two fitted lines (golden fixture);
* the geometric closed form of the expected emitted tokens under a constant
  acceptance rate, and the limits alpha = 0 (plain decoding) and alpha = 1;
* the one-draft decision equals the break-even comparison 1 + alpha_1 >
  cost(2) / cost(1) on both sides of the threshold.
"""

import json
import os

import numpy as np
import pytest

from oracle.depth import break_even_tokens, choose_depth, expected_emitted, linear_window_cost

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "break_even_table.json")


def test_break_even_table_of_the_pages():
    g = json.load(open(GOLDEN))
    for card, (base, per_row) in g["fits_ms"].items():
        cost = [linear_window_cost(base, per_row, r) for r in range(1, 9)]
        got = [round(break_even_tokens(cost, r), 2) for r in g["rows"]]
        assert got == g["break_even_tokens"][card], card


@pytest.mark.parametrize("a", [0.0, 0.3, 0.7, 0.95, 1.0])
def test_expected_emitted_geometric_closed_form(a):
    for k in range(0, 25):
        want = k + 1.0 if a == 1.0 else 1.0 + a * (1.0 - a ** k) / (1.0 - a)
        assert abs(expected_emitted([a] * k, k) - want) <= 1e-12 * want


def test_limits():
    cost = [linear_window_cost(30.5, 6.9, r) for r in range(1, 25)]
    assert choose_depth([0.0] * 23, cost, 23) == (0, 1.0 / 30.5)        # nothing accepted: decode
    k, _ = choose_depth([1.0] * 23, cost, 23)                            # always accepted and
    assert k == 23                                                       # cost(R)/R falls: deepest
    flat = [10.0] * 24                          # rows free: every accepted draft is profit
    assert choose_depth([0.5] * 23, flat, 23)[0] == 23
    # once the running product no longer changes the fp64 sum, ties go to fewer rows
    k, _ = choose_depth([0.01] * 23, flat, 23)
    assert expected_emitted([0.01] * 23, k) == expected_emitted([0.01] * 23, 23) and k < 23


@pytest.mark.parametrize("card", ["strix_halo", "r9700"])
def test_one_draft_decision_is_the_break_even_test(card):
    base, per_row = json.load(open(GOLDEN))["fits_ms"][card]
    cost = [linear_window_cost(base, per_row, r) for r in range(1, 3)]
    be = break_even_tokens(cost, 2)
    for a in np.linspace(0.0, 1.0, 201):
        k, _ = choose_depth([a], cost, 1)
        assert k == (1 if 1.0 + a > be else 0), a


def test_brute_force_rates():
    """k* attains the largest rate among all depths, the smallest such k."""
    g = np.random.default_rng(1900)
    for _ in range(500):
        kmax = int(g.integers(0, 24))
        alpha = g.random(kmax)
        cost = np.cumsum(g.random(kmax + 1) + 0.01) + 5.0
        k, rate = choose_depth(alpha, cost, kmax)
        rates = [expected_emitted(alpha, j) / cost[j] for j in range(kmax + 1)]
        assert rate == max(rates) and k == rates.index(max(rates))
