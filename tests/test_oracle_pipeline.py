"""Pins for the oracle's stage composition (oracle/pipeline.py) on a window
worked out by hand.

[SD] "Speculative decoding on RDNA", §04 and its figure "the penalty history
of verify row i": verify row i is penalised against H_i, the last W tokens
of (prompt || emitted || drafts[0, i)), and the draft's candidates for row
i get the same H_i; §03 "how hipfire does it": the policy (temperature,
top-k, min-p, top-p) runs over the pool of the already-penalised row;
§02/§03: greedy longest-prefix acceptance and the rejection rule.

The window: vocabulary 8, W = 4, k = 2 drafts, repeat 2, frequency 1/4,
presence 1/2, so every penalised logit below is dyadic and exact.  For a
token of count c: l -> (l > 0 ? l / 2 : 2 l) - c/4 - 1/2.

    ctx = [5, 2, 5, 7], drafts = [1, 6]
    H_0 = [5, 2, 5, 7]  counts {5: 2, 2: 1, 7: 1}
    H_1 = [2, 5, 7, 1]  counts {2: 1, 5: 1, 7: 1, 1: 1}
    H_2 = [5, 7, 1, 6]  counts {5: 1, 7: 1, 1: 1, 6: 1}

Each planted mistake (a pool taken before the penalties, q penalised with
H_{i+1}, a drafter that ignores its own earlier drafts, a row penalised with
its neighbour's history) changes a value checked here, so the controls at
the end assert that the check then fails.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.pipeline as pipeline

W = 4
REP, PRES, FREQ = 2.0, 0.5, 0.25
CTX = np.array([5, 2, 5, 7], dtype=np.int32)
DRAFTS = np.array([1, 6], dtype=np.int32)
POOL4 = 4

RAW = np.array([
    [0.5, 1.0, 1.5, 0.25, -1.0, 4.0, 0.0, 2.0],    # row 0, raw argmax 5
    [0.0, 3.0, 1.0, 0.25, -0.5, 0.5, 0.875, 0.0],  # row 1, raw argmax 1
    [1.0, 0.0, 0.0, 0.5, 0.25, 3.0, 2.0, -2.0],    # row 2, raw argmax 5
], dtype=np.float32)

# Row 0 with H_0: 5 (c=2): 4/2 - 1/2 - 1/2 = 1;  2: 3/4 - 3/4 = 0;  7: 1 - 3/4 = 1/4.
# Row 1 with H_1: 1: 3/2 - 3/4 = 3/4;  2: 1/2 - 3/4 = -1/4;  5: 1/4 - 3/4 = -1/2;
#                 7: 0 is not > 0, 2*0 - 3/4 = -3/4.
# Row 2 with H_2: 5: 3/2 - 3/4 = 3/4;  7: -4 - 3/4 = -19/4;  1: 0 - 3/4 = -3/4;
#                 6: 1 - 3/4 = 1/4.
PENALIZED = np.array([
    [0.5, 1.0, 0.0, 0.25, -1.0, 1.0, 0.0, 0.25],
    [0.0, 0.75, -0.25, 0.25, -0.5, -0.5, 0.875, -0.75],
    [1.0, -0.75, 0.0, 0.5, 0.25, 0.75, 0.25, -4.75],
], dtype=np.float32)
# pools of 4 in the order (value desc, id asc): the penalties move every
# row's argmax away from its raw argmax (5, 1, 5 -> 1, 6, 0)
POOL_IDS = np.array([[1, 5, 0, 3], [6, 1, 3, 0], [0, 5, 3, 4]], dtype=np.int32)
POOL_VALS = np.array([[1.0, 1.0, 0.5, 0.25], [0.875, 0.75, 0.25, 0.0], [1.0, 0.75, 0.5, 0.25]],
                     dtype=np.float32)

# The draft's candidates (3 per row), re-scored logits before penalties.
Q_IDS = np.array([[5, 1, 3], [6, 1, 2]], dtype=np.int32)
Q_VALS = np.array([[2.0, 1.0, 0.5], [1.0, 2.0, 0.5]], dtype=np.float32)
# q row 0 with H_0: 5 (c=2): 1 - 1 = 0;  1, 3 not in H_0.
# q row 1 with H_1: 6 not in H_1;  1: 1 - 3/4 = 1/4;  2: 1/4 - 3/4 = -1/2.
Q_PENALIZED = np.array([[0.0, 1.0, 0.5], [1.0, 0.25, -0.5]], dtype=np.float32)

POLICY = dict(temperature=1.0, top_k=2, top_p=1.0, min_p=0.0)


def two_way(delta: float):
    """Probabilities of two candidates whose logits differ by delta >= 0 at T = 1."""
    e = math.exp(-delta)
    return 1.0 / (1.0 + e), e / (1.0 + e)


def run(temperature, u=None, q=True):
    kw = dict(window=W, repeat=REP, presence=PRES, frequency=FREQ, top_k=POLICY["top_k"],
              top_p=POLICY["top_p"], min_p=POLICY["min_p"], pool=POOL4)
    if q:
        kw.update(q_ids=Q_IDS, q_vals=Q_VALS)
    if u is None:
        u = np.zeros((3, 2), dtype=np.float32)
    return pipeline.acceptance_stage(RAW, CTX, DRAFTS, np.asarray(u, dtype=np.float32),
                                     temperature=temperature, **kw)


# u[i][0] is row i's accept test, u[i][1] its replacement or bonus draw.
#   row 0: x = 1, p(1) = 1/2, q(1) = 0.6225 -> 0.75 * 0.6225 = 0.467 < 0.5: accept
#   row 1: x = 6, p(6) = 0.5312, q(6) = 0.6792 -> 0.9 * 0.6792 = 0.611 >= 0.531: reject
#          residual over p's support [6, 1]: (0, 0.4688 - 0.3208) -> token 1
U_SAMPLED = [[0.75, 0.5], [0.9, 0.5], [0.5, 0.25]]


def check_greedy(out):
    np.testing.assert_array_equal(out["penalized"], PENALIZED)
    np.testing.assert_array_equal(out["pool_ids"], POOL_IDS)
    np.testing.assert_array_equal(out["pool_vals"], POOL_VALS)
    # argmax per row 1, 6, 0: both drafts accepted, then the bonus row's argmax
    assert [int(t) for t in out["tokens"]] == [1, 6, 0]


def check_sampled(out):
    np.testing.assert_array_equal(out["penalized"], PENALIZED)
    np.testing.assert_array_equal(out["pool_ids"], POOL_IDS)
    np.testing.assert_array_equal(out["q_penalized"], Q_PENALIZED)
    # p rows: the top 2 of each pool at T = 1
    want_p = [([1, 5], (0.5, 0.5)), ([6, 1], two_way(0.125)), ([0, 5], two_way(0.25))]
    for (ids, probs), (wid, wpr) in zip(out["p_rows"], want_p):
        assert [int(t) for t in ids] == wid
        np.testing.assert_allclose(probs, wpr, rtol=0, atol=1e-7)
    # q rows: the top 2 of the penalised candidates (1, 3 | 6, 1)
    want_q = [([1, 3], two_way(0.5)), ([6, 1], two_way(0.75))]
    for (ids, probs), (wid, wpr) in zip(out["q_rows"], want_q):
        assert [int(t) for t in ids] == wid
        np.testing.assert_allclose(probs, wpr, rtol=0, atol=1e-7)
    assert [int(t) for t in out["tokens"]] == [1, 1]


def test_greedy_window_by_hand():
    out = run(0.0, q=False)
    check_greedy(out)
    # the raw rows' argmax would have rejected the first draft
    assert [int(np.argmax(r)) for r in RAW] == [5, 1, 5]


def test_sampled_window_by_hand():
    check_sampled(run(POLICY["temperature"], U_SAMPLED))


def test_sampled_all_accepted_then_bonus():
    # u10 = 0.5: 0.5 * 0.6792 < 0.5312 accepts row 1; the bonus is drawn from
    # p row 2 = (0: 0.5622, 5: 0.4378) with u21 = 0.25 -> token 0
    out = run(POLICY["temperature"], [[0.75, 0.5], [0.5, 0.5], [0.5, 0.25]])
    assert [int(t) for t in out["tokens"]] == [1, 6, 0]
    out = run(POLICY["temperature"], [[0.75, 0.5], [0.5, 0.5], [0.5, 0.75]])
    assert [int(t) for t in out["tokens"]] == [1, 6, 5]


def draft_kw():
    return dict(vocab=8, window=W, repeat=REP, presence=PRES, frequency=FREQ, **POLICY)


def test_draft_chain_by_hand():
    # d0 ~ q_0 penalised with H_0: (1: 0.6225, 3: 0.3775).  u = 0.5 -> 1.
    # d1 ~ q_1 penalised with last 4 of (ctx || 1) = H_1: (6: 0.6792, 1: 0.3208); u = 0.5 -> 6.
    d = pipeline.draft_chain(Q_IDS, Q_VALS, CTX, np.array([0.5, 0.5], np.float32), **draft_kw())
    assert [int(t) for t in d] == [1, 6]
    # u0 = 0.7 -> d0 = 3; then H_1 = [2, 5, 7, 3] leaves 1 unpenalised:
    # q_1 = (1: 2.0, 6: 1.0) -> (1: 0.7311, 6: 0.2689); u = 0.5 -> 1
    d = pipeline.draft_chain(Q_IDS, Q_VALS, CTX, np.array([0.7, 0.5], np.float32), **draft_kw())
    assert [int(t) for t in d] == [3, 1]


# ---- planted mistakes: each must make the hand-worked checks fail -------------

def test_control_pool_before_penalties(monkeypatch):
    """The pool chosen on the raw logits (penalties applied to the chosen
    values afterwards) picks other candidates."""
    real_topk = pipeline.topk_rows

    def pool_on_raw(pen, k):
        _, ids = real_topk(RAW, k)
        return np.take_along_axis(pen, ids, axis=1), ids

    monkeypatch.setattr(pipeline, "topk_rows", pool_on_raw)
    with pytest.raises(AssertionError):
        check_greedy(run(0.0, q=False))
    with pytest.raises(AssertionError):
        check_sampled(run(POLICY["temperature"], U_SAMPLED))


def test_control_q_penalised_with_next_history(monkeypatch):
    """q row i penalised with H_{i+1} instead of H_i."""
    real = pipeline.penalize_sparse

    def shifted(ids, vals, ctx, drafts, window, repeat, presence, frequency, *, vocab):
        # a dummy first row moves candidate row i to row i + 1, penalised with H_{i+1}
        ids2 = np.vstack([ids[:1], ids])
        vals2 = np.vstack([vals[:1], vals])
        return real(ids2, vals2, ctx, drafts, window, repeat, presence, frequency, vocab=vocab)[1:]

    monkeypatch.setattr(pipeline, "penalize_sparse", shifted)
    with pytest.raises(AssertionError):
        check_sampled(run(POLICY["temperature"], U_SAMPLED))


def test_control_target_rows_with_previous_history(monkeypatch):
    """Target row i penalised with H_{i-1} (a draft entering its own row's history late)."""
    real = pipeline.penalize_dense

    def late(logits, ctx, drafts, window, repeat, presence, frequency):
        out = np.array(logits, dtype=np.float32, copy=True)
        for i in range(out.shape[0]):
            out[i] = real(logits, ctx, drafts[:max(i - 1, 0)], window, repeat, presence,
                          frequency)[i]
        return out

    monkeypatch.setattr(pipeline, "penalize_dense", late)
    with pytest.raises(AssertionError):
        check_greedy(run(0.0, q=False))


def test_control_drafter_ignores_its_drafts(monkeypatch):
    """The drafter penalising q_i with the context only (its own drafts left out)."""
    real = pipeline.penalize_sparse

    def ctx_only(ids, vals, ctx, drafts, window, repeat, presence, frequency, *, vocab):
        return real(ids, vals, ctx, drafts[:0], window, repeat, presence, frequency, vocab=vocab)

    monkeypatch.setattr(pipeline, "penalize_sparse", ctx_only)
    d = pipeline.draft_chain(Q_IDS, Q_VALS, CTX, np.array([0.5, 0.5], np.float32), **draft_kw())
    assert [int(t) for t in d] != [1, 6]


# ---- a token tree ([TREE] "Spend the budget on a tree, not a longer guess") ----
#
# Same vocabulary, penalties and context; three nodes: node 0 (token 1, under
# the root), node 1 (token 6, under node 0), node 2 (token 3, under the root):
# branches [1, 6] and [3].  Row histories (W = 4):
#   row 0 (root)   H = [5, 2, 5, 7]
#   row 1 (node 0) H = last 4 of ctx || [1]    = [2, 5, 7, 1]
#   row 2 (node 1) H = last 4 of ctx || [1, 6] = [5, 7, 1, 6]
#   row 3 (node 2) H = last 4 of ctx || [3]    = [2, 5, 7, 3]
# Rows 0-2 are the chain's RAW rows with row 1's token-6 logit raised to 1,
# so branch [1, 6] is the chain above; row 3 is penalised with its own
# branch, not with the nodes numbered before it.

TREE_TOKENS = np.array([1, 6, 3], dtype=np.int32)
TREE_PARENT = np.array([-1, 0, -1], dtype=np.int32)
TREE_RAW = np.array([
    [0.5, 1.5, 1.0, 0.25, -1.0, 4.0, 0.0, 2.0],
    [0.0, 3.0, 1.0, 0.25, -0.5, 0.5, 1.0, 0.0],
    [1.0, 0.0, 0.0, 0.5, 0.25, 3.0, 2.0, -2.0],
    [0.25, 0.5, 2.0, 1.0, 0.0, 0.75, -0.25, 0.5],
], dtype=np.float32)
# row 0: 5 (c=2): 2 - 1 = 1;  2: 1/2 - 3/4 = -1/4;  7: 1 - 3/4 = 1/4
# row 1: 1: 3/2 - 3/4 = 3/4;  2: -1/4;  5: 1/4 - 3/4 = -1/2;  7: 0 - 3/4 = -3/4
# row 2: 5: 3/4;  7: -4 - 3/4 = -19/4;  1: -3/4;  6: 1 - 3/4 = 1/4
# row 3: 2: 1 - 3/4 = 1/4;  5: 3/8 - 3/4 = -3/8;  7: 1/4 - 3/4 = -1/2;  3: 1/2 - 3/4 = -1/4
TREE_PENALIZED = np.array([
    [0.5, 1.5, -0.25, 0.25, -1.0, 1.0, 0.0, 0.25],
    [0.0, 0.75, -0.25, 0.25, -0.5, -0.5, 1.0, -0.75],
    [1.0, -0.75, 0.0, 0.5, 0.25, 0.75, 0.25, -4.75],
    [0.25, 0.5, 0.25, -0.25, 0.0, -0.375, -0.25, -0.5],
], dtype=np.float32)
TREE_POOL_IDS = np.array([[1, 5, 0, 3], [6, 1, 3, 0], [0, 5, 3, 4], [1, 0, 2, 4]], dtype=np.int32)


def run_tree(temperature, u, top_k=2):
    kw = dict(window=W, repeat=REP, presence=PRES, frequency=FREQ, top_k=top_k, top_p=1.0,
              min_p=0.0, pool=POOL4)
    return pipeline.tree_acceptance_stage(TREE_RAW, CTX, TREE_TOKENS, TREE_PARENT,
                                          np.asarray(u, dtype=np.float32), temperature=temperature,
                                          **kw)


def check_tree(out):
    np.testing.assert_array_equal(out["penalized"], TREE_PENALIZED)
    np.testing.assert_array_equal(out["pool_ids"], TREE_POOL_IDS)


def test_tree_greedy_by_hand():
    out = run_tree(0.0, np.zeros((4, 2)))
    check_tree(out)
    # row argmax 1, 6, 0, 1: node 0 (1) agrees with the root, node 1 (6) with
    # node 0's row, node 2 (3) does not; branch [1, 6], then row 2's argmax 0
    assert [int(t) for t in out["tokens"]] == [1, 6, 0]
    # on the raw rows the root's argmax (5) matches no child
    assert int(np.argmax(TREE_RAW[0])) == 5


# Naive-sampling walk at T = 1, top-2: root p = (1: 0.6225, 5: 0.3775),
# node 0's row (6: 0.5622, 1: 0.4378), node 1's row (0: 0.5622, 5: 0.4378);
# row r draws with u[r][1].
TREE_WALKS = [
    ([[0, 0.5], [0, 0.5], [0, 0.75], [0, 0]], [1, 6, 5]),   # down branch 0, then draw 5
    ([[0, 0.5], [0, 0.5], [0, 0.25], [0, 0]], [1, 6, 0]),
    ([[0, 0.7], [0, 0.0], [0, 0.0], [0, 0]], [5]),          # no child holds 5
    ([[0, 0.5], [0, 0.9], [0, 0.0], [0, 0]], [1, 1]),       # node 0's row draws 1: no child
]


@pytest.mark.parametrize("u,want", TREE_WALKS)
def test_tree_sampled_walk_by_hand(u, want):
    out = run_tree(1.0, u)
    check_tree(out)
    assert [int(t) for t in out["tokens"]] == want


def test_tree_second_branch_by_hand():
    # top-4 at T = 1, root weights e^1.5, e^1, e^0.5, e^0.25 (cumulative 4.48,
    # 7.20, 8.85, 10.13): u = 0.95 draws 3, node 2; its row (1: e^0.5, 0: e^0.25,
    # 2: e^0.25, 4: 1) with u = 0.1 draws 1, which no child holds
    out = run_tree(1.0, [[0, 0.95], [0, 0], [0, 0], [0, 0.1]], top_k=4)
    check_tree(out)
    assert [int(t) for t in out["tokens"]] == [3, 1]


def test_tree_control_branches_as_one_chain(monkeypatch):
    """Row r penalised with ctx || the nodes numbered before it (the tree read
    as one chain) instead of its own branch's path: row 3 changes."""
    def as_chain(logits, ctx, tokens, parent, window, repeat, presence, frequency):
        return pipeline.penalize_dense(logits, ctx, tokens, window, repeat, presence, frequency)

    monkeypatch.setattr(pipeline, "penalize_tree_dense", as_chain)
    with pytest.raises(AssertionError):
        check_tree(run_tree(0.0, np.zeros((4, 2))))


def test_tree_control_pool_before_penalties(monkeypatch):
    real_topk = pipeline.topk_rows

    def pool_on_raw(pen, k):
        _, ids = real_topk(TREE_RAW, k)
        return np.take_along_axis(pen, ids, axis=1), ids

    monkeypatch.setattr(pipeline, "topk_rows", pool_on_raw)
    out = run_tree(0.0, np.zeros((4, 2)))
    with pytest.raises(AssertionError):
        check_tree(out)
    assert [int(t) for t in out["tokens"]] != [1, 6, 0]


def test_tree_control_walk_reads_the_wrong_rows(monkeypatch):
    """The walk given node j's row where it should read row 1 + j."""
    real = pipeline.accept_naive_tree

    def shifted(p_rows, tokens, parent, u):
        return real(p_rows[:1] + p_rows[2:] + p_rows[1:2], tokens, parent, u)

    monkeypatch.setattr(pipeline, "accept_naive_tree", shifted)
    u, want = TREE_WALKS[0]
    assert [int(t) for t in run_tree(1.0, u)["tokens"]] != want
