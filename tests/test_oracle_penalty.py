"""Pins for the penalty oracle.

The per-row history follows the figure "the penalty history of verify row
i" in section 04 of "Speculative decoding on RDNA"; the arithmetic is
checked on dyadic values whose results are exact and worked out by hand,
which also fixes the order of the three penalties.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle.penalty import history, penalize_dense, penalize_sparse, penalize_value


def f32_round(fr: Fraction) -> float:
    """Round a rational to the nearest fp32 (ties to even), by integer arithmetic."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)
    scale = Fraction(2) ** (23 - e)
    m = a * scale
    q, rem = divmod(m.numerator, m.denominator)
    twice = 2 * rem
    if twice > m.denominator or (twice == m.denominator and q % 2 == 1):
        q += 1
    return sign * float(Fraction(q) / scale)


def test_history_rows_grow_by_one_draft():
    ctx = np.array([5, 6, 7, 8, 9], dtype=np.int32)
    d = np.array([1, 2, 3], dtype=np.int32)
    assert history(ctx, d, 0, 4) == [6, 7, 8, 9]
    assert history(ctx, d, 1, 4) == [7, 8, 9, 1]
    assert history(ctx, d, 3, 4) == [9, 1, 2, 3]
    # the bonus row k sees all k drafts; more rows than drafts keep all drafts
    assert history(ctx, d, 5, 4) == [9, 1, 2, 3]
    # H_{i+1} = last W of (H_i || d_i)
    for i in range(3):
        assert history(ctx, d, i + 1, 4) == (history(ctx, d, i, 4) + [int(d[i])])[-4:]
    # window larger than the available context uses everything; W = 0 is empty
    assert history(ctx, d, 2, 100) == [5, 6, 7, 8, 9, 1, 2]
    assert history(ctx, d, 2, 0) == []


def test_hand_values_fix_the_order():
    # repeat 2, frequency 0.25, presence 0.5: every step is exact in fp32
    rep, pres, freq = 2.0, 0.5, 0.25
    assert penalize_value(3.0, 2, rep, pres, freq) == 0.5      # 3/2 - 2*0.25 - 0.5
    assert penalize_value(-3.0, 1, rep, pres, freq) == -6.75   # -3*2 - 0.25 - 0.5
    assert penalize_value(0.0, 3, rep, pres, freq) == -1.25    # 0*2 - 0.75 - 0.5
    # presence once regardless of count; frequency scales with count
    a = penalize_value(8.0, 1, 1.0, 1.5, 0.0)
    b = penalize_value(8.0, 4, 1.0, 1.5, 0.0)
    assert a == b == 6.5
    assert penalize_value(8.0, 4, 1.0, 0.0, 0.5) == 6.0


def test_neutral_parameters_are_identity():
    rng = np.random.default_rng(1)
    for v in rng.standard_normal(50).astype(np.float32):
        assert penalize_value(v, 3, 1.0, 0.0, 0.0) == v


@pytest.mark.parametrize("l,c", [(2.0, 1), (-1.7, 3), (0.3, 2), (-0.0001, 1), (123.456, 5)])
def test_each_operation_rounds_once_in_fp32(l, c):
    rep, pres, freq = np.float32(1.1), np.float32(1.5), np.float32(0.2)
    l = np.float32(l)
    L, REP, PRES, FREQ = (Fraction(float(v)) for v in (l, rep, pres, freq))
    l1 = f32_round(L / REP) if l > 0 else f32_round(L * REP)
    cf = f32_round(Fraction(c) * FREQ)
    l2 = f32_round(Fraction(l1) - Fraction(cf))
    l3 = f32_round(Fraction(l2) - PRES)
    assert penalize_value(l, c, rep, pres, freq) == np.float32(l3)


def test_dense_touches_only_history_tokens():
    V = 50
    logits = np.linspace(-5, 5, 3 * V, dtype=np.float32).reshape(3, V)
    ctx = np.array([4, 4, 10, 60, -1, 7], dtype=np.int32)  # 60 and -1 are out of range
    d = np.array([10, 11], dtype=np.int32)
    out = penalize_dense(logits, ctx, d, window=6, repeat=2.0, presence=0.5, frequency=0.25)
    changed = [set(np.nonzero(out[i] != logits[i])[0]) for i in range(3)]
    assert changed[0] == {4, 10, 7}
    assert changed[1] == {4, 10, 7}          # H_1 = [4, 10, 60, -1, 7, 10]
    assert changed[2] == {10, 7, 11}         # H_2 = [10, 60, -1, 7, 10, 11]
    # token 10 is counted twice in row 1 (ctx and draft 0)
    assert out[1, 10] == penalize_value(logits[1, 10], 2, 2.0, 0.5, 0.25)
    assert out[0, 10] == penalize_value(logits[0, 10], 1, 2.0, 0.5, 0.25)


def test_sparse_matches_dense_on_the_same_ids():
    rng = np.random.default_rng(3)
    V = 40
    logits = rng.standard_normal((4, V)).astype(np.float32) * 3
    ctx = rng.integers(0, V, 30).astype(np.int32)
    d = rng.integers(0, V, 3).astype(np.int32)
    dense = penalize_dense(logits, ctx, d, 16, 1.1, 1.5, 0.2)
    ids = np.stack([rng.permutation(V)[:8] for _ in range(4)]).astype(np.int32)
    vals = np.take_along_axis(logits, ids.astype(np.int64), axis=1)
    sparse = penalize_sparse(ids, vals, ctx, d, 16, 1.1, 1.5, 0.2, vocab=V)
    assert np.array_equal(sparse, np.take_along_axis(dense, ids.astype(np.int64), axis=1))



def test_sparse_ignores_ids_outside_the_vocabulary():
    """History tokens outside [0, vocab) are ignored for sparse rows as for
    dense ones, so slots holding such ids (empty slots are negative) keep
    their logits even when the same id sits in the history."""
    V = 12
    ctx = np.array([-3, V + 2, 5, 5, -1, V], dtype=np.int32)
    d = np.array([5], dtype=np.int32)
    ids = np.array([[-3, V + 2, 5, 6, -1, V]] * 2, dtype=np.int32)
    vals = np.array([[2.0, -1.0, 3.0, 4.0, 0.5, 1.5]] * 2, dtype=np.float32)
    out = penalize_sparse(ids, vals, ctx, d, 16, 1.1, 1.5, 0.2, vocab=V)
    keep = np.array([0, 1, 3, 4, 5])
    assert np.array_equal(out[:, keep], vals[:, keep])
    dense = np.zeros((2, V), dtype=np.float32)
    dense[:, 5] = 3.0
    want = penalize_dense(dense, ctx, d, 16, 1.1, 1.5, 0.2)[:, 5]
    assert np.array_equal(out[:, 2], want)
    assert out[0, 2] != out[1, 2]  # row 1 also sees the draft: count 3 against 2

# ----------------------------------------------------------- token trees


def test_tree_histories_hand_worked():
    """Row 0 (root) sees the context; node j's row sees context || its path."""
    from oracle.penalty import tree_history

    ctx, tokens, parent = [5, 6], [7, 8, 9, 4], [-1, 0, -1, 1]
    assert [tree_history(ctx, tokens, parent, r, 3) for r in range(5)] == \
        [[5, 6], [5, 6, 7], [6, 7, 8], [5, 6, 9], [7, 8, 4]]
    assert [tree_history(ctx, tokens, parent, r, 0) for r in range(5)] == [[]] * 5
    # a parent outside [-1, j) ends the path as the root would
    assert tree_history(ctx, [7, 8], [1, 5], 2, 10) == [5, 6, 8]


def test_chain_tree_gives_the_chain_histories():
    from oracle.penalty import tree_history

    g = np.random.default_rng(1970)
    for _ in range(100):
        ctx = list(g.integers(0, 50, size=int(g.integers(0, 80))))
        k = int(g.integers(0, 20))
        drafts = g.integers(0, 50, size=k)
        W = int(g.integers(0, 40))
        chain_parent = list(range(-1, k - 1))
        for r in range(k + 1):
            assert tree_history(ctx, drafts, chain_parent, r, W) == history(np.array(ctx), drafts, r, W)


def test_tree_penalties_equal_chain_penalties_on_a_chain():
    from oracle.penalty import penalize_tree_dense, penalize_tree_sparse

    g = np.random.default_rng(1971)
    V, k = 300, 6
    logits = (g.standard_normal((k + 1, V)) * 3).astype(np.float32)
    ctx = g.integers(0, V, size=120)
    drafts = g.integers(0, V, size=k)
    parent = np.arange(-1, k - 1)
    args = (40, 1.1, 1.5, 0.2)
    assert np.array_equal(penalize_tree_dense(logits, ctx, drafts, parent, *args),
                          penalize_dense(logits, ctx, drafts, *args))
    ids = g.integers(0, V, size=(k + 1, 8)).astype(np.int32)
    vals = logits[:, :8].copy()
    assert np.array_equal(penalize_tree_sparse(ids, vals, ctx, drafts, parent, *args, vocab=V),
                          penalize_sparse(ids, vals, ctx, drafts, *args, vocab=V))
