"""GPU parity of penalize_rows: bit identity with the fp32 oracle.

Histories follow the figure "the penalty history of verify row i" in section
04 of "Speculative decoding on RDNA"; the LM-head case uses a 2048-token
prompt plus 32 emitted tokens with a quarter of the positions drawn from the
rows' highest-logit tokens, so the penalties actually reach the pool.
"""

import numpy as np
import pytest

import verify_sampling_amd as vs
from gpu_common import dev, host
from oracle.penalty import penalize_dense, penalize_sparse
from synth import VOCAB, draft_candidates, logits, penalty_history

pytestmark = pytest.mark.gpu
P = dict(repeat=1.1, presence=1.5, frequency=0.2)


def hot_tokens(x, n=64):
    return np.unique(np.argsort(-x, axis=1)[:, :n])


def run_dense(x, ctx, drafts, window, **p):
    t = dev(x)
    vs.penalize_rows(t, dev(ctx), dev(drafts), window=window, **p)
    return host(t)


def test_lm_head_rows_dense():
    x = logits(1600, (4, VOCAB))
    ctx = penalty_history(1601, VOCAB, 2048, 32, hot_tokens(x))
    drafts = np.argsort(-x[:3], axis=1)[:, 1].astype(np.int32)
    got = run_dense(x, ctx, drafts, 64, **P)
    want = penalize_dense(x, ctx, drafts, 64, **P)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert (got != x).sum() > 4 * 20  # the window touched many logits


def test_draft_candidates_sparse():
    x = logits(1602, (4, VOCAB))
    ctx = penalty_history(1603, VOCAB, 2048, 32, hot_tokens(x))
    ids, vals = draft_candidates(1604, x[:3], 8)
    drafts = ids[:, 0].copy()
    t = dev(vals)
    vs.penalize_rows(t, dev(ctx), dev(drafts), window=64, ids=dev(ids), vocab=VOCAB, **P)
    want = penalize_sparse(ids, vals, ctx, drafts, 64, **P, vocab=VOCAB)
    assert np.array_equal(host(t).view(np.uint32), want.view(np.uint32))


@pytest.mark.parametrize("ctx_len,n_drafts,window,rows", [
    (0, 3, 64, 4), (10, 3, 64, 4), (5000, 0, 4096, 2), (100, 5, 3, 7), (64, 2, 1, 3),
    (300, 10, 200, 12), (600, 4, 128, 5), (600, 4, 129, 5), (3000, 7, 1000, 8),
    (4090, 9, 4096, 10)])
def test_windows_and_edges(ctx_len, n_drafts, window, rows):
    """Dense and sparse rows.  Dense histories of up to 128 tokens are
    scanned, longer ones counted in a hash table (the threshold sits between
    the 128- and 129-token windows)."""
    V = 3000
    g = np.random.default_rng(ctx_len + 7 * window + rows)
    x = logits(1605 + rows, (rows, V))
    x[:, :50] = 0.0
    x[:, 50:60] = -0.0
    ctx = g.integers(-5, V + 5, ctx_len).astype(np.int32)   # some ids out of range
    ctx[::3] = g.integers(0, 40, len(ctx[::3]))               # repeats
    drafts = g.integers(0, 60, n_drafts).astype(np.int32)
    got = run_dense(x, ctx, drafts, window, **P)
    want = penalize_dense(x, ctx, drafts, window, **P)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # sparse: slots holding repeated, single, absent and out-of-range ids
    ids = np.where(g.random((rows, 16)) < 0.5, g.integers(0, 40, (rows, 16)),
                   g.integers(-3, V + 3, (rows, 16))).astype(np.int32)
    vals = logits(1615 + rows, (rows, 16))
    t = dev(vals)
    vs.penalize_rows(t, dev(ctx), dev(drafts), window=window, ids=dev(ids), vocab=V, **P)
    want = penalize_sparse(ids, vals, ctx, drafts, window, **P, vocab=V)
    assert np.array_equal(host(t).view(np.uint32), want.view(np.uint32))


def test_long_history_of_one_token():
    """A 4096-token history of a single id: in dense rows one hash slot
    takes every occurrence; in sparse rows counted per slot."""
    V = 1000
    x = logits(1620, (4, V))
    ctx = np.full(5000, 7, dtype=np.int32)
    drafts = np.array([7, 8, 7], dtype=np.int32)
    got = run_dense(x, ctx, drafts, 4096, **P)
    want = penalize_dense(x, ctx, drafts, 4096, **P)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    ids = np.tile(np.array([7, 8, 9, 7], dtype=np.int32), (4, 1))
    vals = logits(1621, (4, 4))
    t = dev(vals)
    vs.penalize_rows(t, dev(ctx), dev(drafts), window=4096, ids=dev(ids), vocab=V, **P)
    want = penalize_sparse(ids, vals, ctx, drafts, 4096, **P, vocab=V)
    assert np.array_equal(host(t).view(np.uint32), want.view(np.uint32))


def test_window_zero_and_neutral_are_noops():
    x = logits(1606, (3, 2000))
    ctx = np.arange(100, dtype=np.int32)
    d = np.array([1, 2], dtype=np.int32)
    assert np.array_equal(run_dense(x, ctx, d, 0, **P).view(np.uint32), x.view(np.uint32))
    neutral = dict(repeat=1.0, presence=0.0, frequency=0.0)
    assert np.array_equal(run_dense(x, ctx, d, 64, **neutral).view(np.uint32), x.view(np.uint32))


def tree_cases():
    """(ctx, tokens, parent) trees: prompt-lookup trees over copied lines, a
    chain, a 63-node tree, a root-only tree and malformed parents."""
    from synth import lookup_context

    V = 4096
    ctx = lookup_context(1620, 6000, vocab=V)
    out = []
    for e, n, B, D in ((2000, 3, 3, 8), (4100, 2, 4, 6), (5990, 3, 3, 8)):
        tk, par = vs.lookup_tree(ctx[:e], n, B, D, 24)
        out.append((ctx[:e], tk, par))
    g = np.random.default_rng(1621)
    chain = g.integers(0, V, size=10).astype(np.int32)
    out.append((ctx[:300], chain, np.arange(-1, 9, dtype=np.int32)))
    big_par = np.array([-1] + [int(g.integers(-1, j)) for j in range(1, 63)], dtype=np.int32)
    out.append((ctx[:700], g.integers(0, V, size=63).astype(np.int32), big_par))
    out.append((ctx[:50], np.zeros(0, dtype=np.int32), np.zeros(0, dtype=np.int32)))
    bad = np.array([-1, 5, 0, 3, -7], dtype=np.int32)   # parents outside [-1, j) end the path
    out.append((ctx[:90], g.integers(0, V, size=5).astype(np.int32), bad))
    return out


@pytest.mark.parametrize("case", range(7))
@pytest.mark.parametrize("window", [64, 5, 4096])
def test_tree_rows_dense_and_sparse(case, window):
    """penalize_tree_rows: row 0 sees the context, row 1 + j the context and
    node j's root path ("Spend the budget on a tree" of the verify-slack
    page); bit-identical to the oracle, dense and sparse."""
    from oracle.penalty import penalize_tree_dense, penalize_tree_sparse

    ctx, tk, par = tree_cases()[case]
    V = 4096
    rows = len(tk) + 1
    x = logits(1630 + case, (rows, V))
    t = dev(x)
    vs.penalize_tree_rows(t, dev(ctx), dev(tk), dev(par), window=window, **P)
    want = penalize_tree_dense(x, ctx, tk, par, window, **P)
    assert np.array_equal(host(t).view(np.uint32), want.view(np.uint32))
    g = np.random.default_rng(1640 + case)
    ids = np.where(g.random((rows, 8)) < 0.5, g.choice(ctx[-64:], size=(rows, 8)),
                   g.integers(0, V, size=(rows, 8))).astype(np.int32)
    vals = logits(1650 + case, (rows, 8))
    t = dev(vals)
    vs.penalize_tree_rows(t, dev(ctx), dev(tk), dev(par), window=window, ids=dev(ids), vocab=V, **P)
    want = penalize_tree_sparse(ids, vals, ctx, tk, par, window, **P, vocab=V)
    assert np.array_equal(host(t).view(np.uint32), want.view(np.uint32))


def test_sparse_rows_wider_than_one_chunk():
    """300 candidate slots per row: two chunks of slots (256, then 44), each
    slot's count split over several threads."""
    V = 2000
    g = np.random.default_rng(1625)
    ctx = g.integers(0, V, 3000).astype(np.int32)
    ctx[::2] = g.integers(0, 30, len(ctx[::2]))
    drafts = g.integers(0, 30, 4).astype(np.int32)
    ids = np.where(g.random((5, 300)) < 0.5, g.integers(0, 30, (5, 300)),
                   g.integers(-2, V + 2, (5, 300))).astype(np.int32)
    vals = logits(1626, (5, 300))
    for window in (64, 1000):
        t = dev(vals)
        vs.penalize_rows(t, dev(ctx), dev(drafts), window=window, ids=dev(ids), vocab=V, **P)
        want = penalize_sparse(ids, vals, ctx, drafts, window, **P, vocab=V)
        assert np.array_equal(host(t).view(np.uint32), want.view(np.uint32)), window
