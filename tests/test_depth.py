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


@pytest.mark.gpu
def test_matches_oracle_on_a_cost_table_timed_on_the_gpu():
    """[SD] §05: the depth is chosen on the measured cost of a verify window.
    Here the cost of R = 1..24 rows is the median of 10 timed
    verify_gemv_rows calls (after 2 warm-ups) on a 24576 x 4096 bf16 matrix
    (a fused gate|up projection) on this GPU; the library's chooser and the
    oracle must return the same depth and the same fp64 rate on it."""
    import torch

    from synth import torch_bf16_weights

    dev = "cuda:0"
    W = torch_bf16_weights((24576, 4096), 1970, dev)
    X = torch.randn((24, 4096), generator=torch.Generator().manual_seed(1971)).to(dev)
    Y = torch.empty((24, 24576), dtype=torch.float32, device=dev)
    ws = torch.empty(max(vs.verify_gemv_rows_workspace_bytes(24576, 4096, r) for r in range(1, 25)),
                     dtype=torch.uint8, device=dev)
    cost = []
    for r in range(1, 25):
        times = []
        for it in range(12):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            vs.verify_gemv_rows(W, X[:r], Y[:r], workspace=ws)
            e1.record()
            e1.synchronize()
            if it >= 2:
                times.append(e0.elapsed_time(e1))
        cost.append(float(np.median(times)))
    print("cost ms, R = 1..24:", [round(c, 4) for c in cost])
    assert all(c > 0 and math.isfinite(c) for c in cost)
    g = np.random.default_rng(1972)
    profiles = [[a] * 23 for a in (0.0, 0.3, 0.5, 0.7, 0.8, 0.9, 0.95, 0.99, 1.0)]
    profiles += [list(0.95 * 0.9 ** np.arange(23)), list(g.random(23)), list(g.random(23) ** 0.2)]
    for alpha in profiles:
        for kmax in (3, 7, 15, 23):
            a, c = alpha[:kmax], cost[:kmax + 1]
            assert vs.choose_depth(a, c) == choose_depth(a, c, kmax), (alpha[0], kmax)
