"""GPU parity of sample_policy_rows against the oracle policy and draw.

Ids and lengths must match exactly; probabilities (fp64 arithmetic rounded
once to fp32 on both sides, with exp the only function evaluated by
different libraries) within 1 fp32 ulp; drawn tokens exactly, except where
the draw's target lies within 1e-6 of a cumulative boundary (listed).
"""

import itertools

import numpy as np
import pytest

import verify_sampling_amd as vs
from gpu_common import dev, host, ulp_diff_f32
from oracle.policy import draw, policy_row
from oracle.topk import topk_rows
from synth import correlated_logits, logits, uniforms

pytestmark = pytest.mark.gpu


def run(vals, ids, u, **cfg):
    d_ids, d_probs, d_len, drawn = vs.sample_policy_rows(dev(vals), dev(ids), u=dev(u), **cfg)
    return host(d_ids), host(d_probs), host(d_len), host(drawn)


def near_tie(probs, u):
    c = np.cumsum(np.asarray(probs, dtype=np.float64))
    return np.min(np.abs(float(u) * c[-1] - c)) <= 1e-6 if len(c) else False


def compare(vals, ids, u, **cfg):
    gi, gp, gl, gd = run(vals, ids, u, **cfg)
    ties = []
    for r in range(vals.shape[0]):
        oi, op = policy_row(vals[r], ids[r], **cfg)
        L = len(oi)
        assert gl[r] == L, (r, gl[r], L)
        assert np.array_equal(gi[r, :L], oi), r
        assert (ulp_diff_f32(gp[r, :L], op) <= 1).all(), r
        assert (gi[r, L:] == -1).all() and (gp[r, L:] == 0).all()
        want = int(oi[draw(op, u[r])]) if L else -1
        if gd[r] != want:
            assert near_tie(op, u[r]), (r, gd[r], want)
            ties.append(r)
    return ties


CFG = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)


def test_target_pools():
    x = logits(1700, (256, 4096))
    pv, pi = topk_rows(x, 64)
    assert compare(pv, pi, uniforms(1701, 256), **CFG) == []


def test_draft_candidates_unsorted():
    p = logits(1702, (128, 4096))
    q = correlated_logits(p, 0.9, 1703)
    g = np.random.default_rng(1704)
    ids = np.stack([g.permutation(4096)[:8] for _ in range(128)]).astype(np.int32)
    vals = np.take_along_axis(q, ids.astype(np.int64), axis=1)
    compare(vals, ids, uniforms(1705, 128), **CFG)


@pytest.mark.parametrize("T,top_k,top_p,min_p", list(itertools.product(
    [0.0, 0.7, 1.5], [-1, 0, 1, 5], [0.0, 0.5, 0.95, 1.0], [0.0, 0.05, 1.0])))
def test_parameter_grid(T, top_k, top_p, min_p):
    x = logits(1706, (16, 2048))
    pv, pi = topk_rows(x, 64)
    compare(pv, pi, uniforms(1707, 16), temperature=T, top_k=top_k, top_p=top_p, min_p=min_p)


def test_special_values_and_empty_slots():
    nan, inf = np.nan, np.inf
    vals = np.array([
        [1.0, nan, 2.0, -inf, 2.0, 0.0, -0.0, 3.0],
        [inf, 1.0, inf, 0.0, nan, 2.0, 2.0, 2.0],
        [-inf, -inf, nan, -inf, nan, -inf, -inf, -inf],
        [nan] * 8,
        [1.0, 2.0, 3.0, 4.0, 5.0, 6.0, 7.0, 8.0],
        [5.0] * 8,
    ], dtype=np.float32)
    ids = np.array([
        [5, 6, 9, 8, 3, 1, 2, 7],
        [4, 5, 2, 1, 0, 9, 8, 7],
        [1, 2, 3, 4, 5, 6, 7, 8],
        [9, 8, 7, 6, 5, 4, 3, 2],
        [-1, 10, -1, 11, 12, -1, 13, -1],   # empty slots
        [-1] * 8,                           # nothing at all
    ], dtype=np.int32)
    compare(vals, ids, uniforms(1708, 6), **CFG)
    compare(vals, ids, uniforms(1709, 6), temperature=1.0, top_k=0, top_p=1.0, min_p=0.0)


def test_presorted_and_shuffled_pools_agree():
    """A pool already in pool order (as topk_rows leaves it) skips the sort;
    the same candidates in any other order give the same distribution and
    draw bit for bit.  NaN, -inf and trailing empty slots included."""
    x = logits(1710, (64, 4096))
    x[0, :4000] = np.nan
    x[1, ::2] = -np.inf
    x[2, :] = 1.5
    pv, pi = topk_rows(x, 64)
    pi = pi.copy()
    pi[3, 40:] = -1          # trailing empty slots
    pi[4, 1:] = -1
    u = uniforms(1711, 64)
    for cfg in (CFG, dict(temperature=1.0, top_k=0, top_p=0.9, min_p=0.0)):
        a = run(pv, pi, u, **cfg)
        g = np.random.default_rng(1712)
        perm = np.stack([g.permutation(64) for _ in range(64)])
        b = run(np.take_along_axis(pv, perm, axis=1), np.take_along_axis(pi, perm, axis=1), u, **cfg)
        for ga, gb in zip(a, b):
            assert np.array_equal(np.asarray(ga).view(np.uint32), np.asarray(gb).view(np.uint32))
        compare(pv, pi, u, **cfg)
