"""Pins for oracle/tree_attention.py (tree attention mask over context KV and
scratch slots; commit of the accepted branch), each independent of the
oracle's own formulation:
  * a hand-worked tree whose keys are all equal, so every row's output is
    the plain mean of the values it may see;
  * a chain tree against causal attention over the concatenated sequence,
    built with an explicit lower-triangular mask and scipy's softmax;
  * every row of random trees against plain attention over the sequence
    context || the slots on its root path, the path walked here;
  * changing a slot outside a row's ancestor set leaves the row bit for bit
    unchanged, changing an ancestor does not;
  * grouped heads read the right KV head; malformed parents; the commit.
"""

from __future__ import annotations

import numpy as np
import pytest
from scipy.special import softmax

from oracle.tree_attention import bf16_to_f64, commit_branch, row_slots, tree_attention
from synth import f32_to_bf16_bits


def bf16(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_hand_worked_equal_scores_give_means():
    # one head, D = 2, one context position; root with two children
    # ([TREE] "Spend the budget on a tree": the children see the root, not each other)
    k_cache = bf16(np.ones((1, 1, 2)))
    v_cache = bf16([[[1.0, 0.0]]])
    k_scr = bf16(np.ones((1, 3, 2)))
    v_scr = bf16([[[0.0, 1.0], [2.0, 2.0], [4.0, -4.0]]])
    q = np.array([[[0.3, -0.7]], [[1.5, 2.5]], [[-3.0, 0.25]]], dtype=np.float32)
    out, _ = tree_attention(q, k_cache, v_cache, 1, k_scr, v_scr, [-1, -1], scale=0.5)
    np.testing.assert_allclose(out[0, 0], [0.5, 0.5], rtol=0, atol=1e-15)        # ctx, root
    np.testing.assert_allclose(out[1, 0], [1.0, 1.0], rtol=0, atol=1e-15)        # ctx, root, node 0
    np.testing.assert_allclose(out[2, 0], [5.0 / 3.0, -1.0], rtol=0, atol=1e-15)  # ctx, root, node 1


def test_hand_worked_two_keys_weights_two_to_one():
    # scores ln 2 and 0: weights 2/3 and 1/3
    k_cache = bf16([[[1.0]]])
    v_cache = bf16([[[3.0]]])
    k_scr = bf16([[[0.0]]])
    v_scr = bf16([[[-3.0]]])
    q = np.array([[[np.log(2.0)]]], dtype=np.float32)
    out, _ = tree_attention(q, k_cache, v_cache, 1, k_scr, v_scr, [], scale=1.0)
    assert abs(out[0, 0, 0] - (2.0 - 1.0)) < 1e-7  # 3 * 2/3 - 3 * 1/3


def random_case(seed, R, Hq, Hkv, D, ctx_len, L=None):
    g = np.random.default_rng(seed)
    L = L or ctx_len + R + 4
    q = g.standard_normal((R, Hq, D)).astype(np.float32)
    kc = bf16(g.standard_normal((Hkv, L, D)))
    vc = bf16(g.standard_normal((Hkv, L, D)))
    ks = bf16(g.standard_normal((Hkv, R, D)))
    vs = bf16(g.standard_normal((Hkv, R, D)))
    return q, kc, vc, ks, vs


def test_chain_is_causal_attention():
    R, Hq, Hkv, D, ctx = 9, 4, 2, 16, 13
    q, kc, vc, ks, vs = random_case(2100, R, Hq, Hkv, D, ctx)
    scale = 1.0 / np.sqrt(D)
    parent = list(range(-1, R - 2))
    out, _ = tree_attention(q, kc, vc, ctx, ks, vs, parent, scale)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        K = np.concatenate([bf16_to_f64(kc[g, :ctx]), bf16_to_f64(ks[g])])  # [ctx + R][D]
        V = np.concatenate([bf16_to_f64(vc[g, :ctx]), bf16_to_f64(vs[g])])
        Q = q[:, h].astype(np.float64)
        S = scale * (Q @ K.T)                                   # [R][ctx + R]
        mask = np.tril(np.ones((R, R), dtype=bool))             # slot j visible to row r iff j <= r
        full = np.concatenate([np.ones((R, ctx), dtype=bool), mask], axis=1)
        P = softmax(np.where(full, S, -np.inf), axis=1)
        np.testing.assert_allclose(out[:, h], P @ V, rtol=1e-12, atol=1e-12)


def plain_path_attention(q, kc, vc, ks, vs, ctx, parent, r, h, group, scale):
    """Attention of row r, head h over context || the slots on its root path,
    the path found by walking parents."""
    path = []
    if r > 0:
        j = r - 1
        path.append(1 + j)
        while True:
            p = int(parent[j])
            if not (-1 < p < j):
                break
            path.append(1 + p)
            j = p
    slots = [0] + path[::-1]
    g = h // group
    K = np.concatenate([bf16_to_f64(kc[g, :ctx]), bf16_to_f64(ks[g, slots])])
    V = np.concatenate([bf16_to_f64(vc[g, :ctx]), bf16_to_f64(vs[g, slots])])
    return softmax(scale * (K @ q[r, h].astype(np.float64))) @ V


@pytest.mark.parametrize("seed", [2110, 2111, 2112])
def test_every_row_is_attention_over_its_path(seed):
    g = np.random.default_rng(seed)
    n = 24
    parent = [-1] + [int(g.integers(-1, j)) for j in range(1, n)]
    R, Hq, Hkv, D, ctx = n + 1, 4, 1, 8, 31
    q, kc, vc, ks, vs = random_case(seed + 50, R, Hq, Hkv, D, ctx)
    out, s_abs = tree_attention(q, kc, vc, ctx, ks, vs, parent, 0.3)
    for r in range(R):
        for h in range(Hq):
            want = plain_path_attention(q, kc, vc, ks, vs, ctx, parent, r, h, Hq // Hkv, 0.3)
            np.testing.assert_allclose(out[r, h], want, rtol=1e-12, atol=1e-12)
    assert (s_abs >= np.abs(out) - 1e-12).all()


def test_only_ancestors_matter():
    # 3 branches x depth 8 (the 24-node tree), one context position
    parent = []
    for b in range(3):
        for d in range(8):
            parent.append(-1 if d == 0 else len(parent) - 1)
    R, Hq, Hkv, D, ctx = 25, 2, 1, 8, 5
    q, kc, vc, ks, vs = random_case(2120, R, Hq, Hkv, D, ctx)
    out, _ = tree_attention(q, kc, vc, ctx, ks, vs, parent, 0.4)
    r = 1 + 10                  # node 10: branch 1, depth 3 -> slots 0, 9, 10, 11
    assert row_slots(parent, r) == [0, 9, 10, 11]
    for slot, changes in ((5, False), (20, False), (12, False), (9, True), (0, True), (11, True)):
        ks2, vs2 = ks.copy(), vs.copy()
        vs2[:, slot] ^= np.uint16(0x0040)  # flip a mantissa bit of the value
        out2, _ = tree_attention(q, kc, vc, ctx, ks2, vs2, parent, 0.4)
        assert (not np.array_equal(out2[r], out[r])) == changes, slot


def test_grouped_heads_read_their_kv_head():
    R, Hq, Hkv, D, ctx = 3, 6, 3, 8, 7
    q, kc, vc, ks, vs = random_case(2130, R, Hq, Hkv, D, ctx)
    out, _ = tree_attention(q, kc, vc, ctx, ks, vs, [-1, 0], 0.5)
    for h in range(Hq):
        g = h // 2
        one, _ = tree_attention(q[:, h:h + 1], kc[g:g + 1], vc[g:g + 1], ctx, ks[g:g + 1], vs[g:g + 1],
                                [-1, 0], 0.5)
        np.testing.assert_array_equal(out[:, h], one[:, 0])


def test_malformed_parent_sees_only_the_root():
    assert row_slots([-1, 5, 0], 2) == [0, 2]      # node 1's parent 5 is not below it
    assert row_slots([-1, 5, 0], 3) == [0, 1, 3]
    assert row_slots([-1, -7], 2) == [0, 2]


def test_commit_copies_the_accepted_branch():
    R, Hkv, D, ctx, L = 6, 2, 4, 10, 20
    _, kc, vc, ks, vs = random_case(2140, R, 2, Hkv, D, ctx, L)
    path = [0, 2, 5]
    kc2, vc2 = commit_branch(kc, vc, ctx, ks, vs, path)
    for i, s in enumerate(path):
        assert np.array_equal(kc2[:, ctx + i], ks[:, s]) and np.array_equal(vc2[:, ctx + i], vs[:, s])
    untouched = [p for p in range(L) if not ctx <= p < ctx + len(path)]
    assert np.array_equal(kc2[:, untouched], kc[:, untouched])
    assert np.array_equal(vc2[:, untouched], vc[:, untouched])
