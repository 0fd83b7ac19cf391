"""The library's prompt-lookup tree drafter (host code) against the oracle:
identical trees on random contexts (small vocabularies, so n-grams recur
many times) and on a long context; host-side argument checks.  No GPU."""

import numpy as np
import pytest

import verify_sampling_amd as vs
from oracle.lookup import lookup_tree


def test_matches_oracle_random():
    g = np.random.default_rng(1960)
    for _ in range(2000):
        ctx = g.integers(0, int(g.integers(2, 9)), size=int(g.integers(0, 300)))
        n, B, D = int(g.integers(1, 5)), int(g.integers(1, 6)), int(g.integers(1, 11))
        budget = int(g.integers(1, 64))
        tok, par = vs.lookup_tree(ctx, n, B, D, budget)
        want_t, want_p = lookup_tree(list(ctx), n, B, D, budget)
        assert list(tok) == want_t and list(par) == want_p


def test_matches_oracle_long_context_with_copied_lines():
    from synth import lookup_context

    ctx = lookup_context(1961, 32768)
    for n in (2, 3, 4):
        tok, par = vs.lookup_tree(ctx, n, 3, 8, 24)
        want_t, want_p = lookup_tree(list(ctx), n, 3, 8, 24)
        assert list(tok) == want_t and list(par) == want_p


def test_rejects_bad_arguments():
    with pytest.raises(vs.VerifySamplingError):
        vs.lookup_tree([1, 2, 3], 0, 3, 8)
    with pytest.raises(vs.VerifySamplingError):
        vs.lookup_tree([1, 2, 3], 2, 3, 8, max_nodes=64)
    assert [len(a) for a in vs.lookup_tree([1, 2], 2, 3, 8)] == [0, 0]   # no earlier match
