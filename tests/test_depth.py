"""The library's depth chooser (host code) against the oracle: same depth and
the same fp64 rate bit for bit, on the pages' fits and on random inputs; and
host-side argument checks.  No GPU needed."""

import json
import math
import os

import numpy as np
import pytest

import verify_sampling_amd as vs
from oracle.depth import choose_depth, linear_window_cost

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "break_even_table.json")


def test_matches_oracle_on_the_pages_fits():
    fits = json.load(open(GOLDEN))["fits_ms"]
    for base, per_row in fits.values():
        cost = [linear_window_cost(base, per_row, r) for r in range(1, 9)]
        for a in np.linspace(0.0, 1.0, 101):
            alpha = [float(a)] * 7
            assert vs.choose_depth(alpha, cost) == choose_depth(alpha, cost, 7)


def test_matches_oracle_on_random_inputs():
    g = np.random.default_rng(1910)
    for _ in range(3000):
        kmax = int(g.integers(0, 64))
        alpha = list(g.random(kmax) ** float(g.choice([0.2, 1.0, 3.0])))
        cost = list(np.cumsum(g.random(kmax + 1) * float(g.choice([0.1, 1.0, 10.0])) + 1e-3) + 1.0)
        k, rate = vs.choose_depth(alpha, cost)
        k0, rate0 = choose_depth(alpha, cost, kmax)
        assert k == k0 and rate == rate0


def test_rejects_bad_arguments():
    with pytest.raises(vs.VerifySamplingError):
        vs.choose_depth([1.5], [1.0, 2.0])          # alpha outside [0, 1]
    with pytest.raises(vs.VerifySamplingError):
        vs.choose_depth([0.5], [1.0, 0.0])          # cost must be > 0
    with pytest.raises(vs.VerifySamplingError):
        vs.choose_depth([0.5], [1.0, math.nan])
    with pytest.raises(vs.VerifySamplingError):
        vs.choose_depth([0.5] * 64, [1.0] * 65)     # more than VS_MAX_DRAFTS
    assert vs.choose_depth([], [3.0]) == (0, 1.0 / 3.0)
