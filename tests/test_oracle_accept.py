"""Pins for the acceptance oracle.

* the worked example of section 01 of "Speculative decoding on RDNA"
  (golden fixture), and the "at least one token" invariant stated there;
* an exact enumeration over a grid of uniforms showing the emitted token
  follows p (section 03: the emitted tokens follow p exactly);
* the point-mass draft of section 06 (accept with probability p(c), else a
  draw from p without c);
* the 200,000-trial chi-square test of section 03, with its control: the
  same test must fail when the rejection replacement is drawn from p
  instead of the residual (the mistake is planted in the oracle here, on
  the CPU);
* the token tree against a brute-force enumeration of root paths.
"""

import json
import os

import numpy as np
import pytest

import oracle.accept as acc
from oracle.accept import accept_greedy_chain, accept_greedy_tree, accept_sampled
from oracle.policy import draw, policy_row
from stats import chi2_pvalue
from synth import chain_greedy_case, correlated_logits, logits, tree_greedy_case, uniforms

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_worked_example_window():
    with open(os.path.join(GOLDEN, "worked_example_window.json")) as f:
        g = json.load(f)
    v = g["vocab"]
    drafts = [v[w] for w in g["drafts"]]
    argmax = [v[w] for w in g["target_argmax"]]
    out = accept_greedy_chain(argmax, drafts)
    assert out == [v[w] for w in g["expected_tokens"]]
    assert len(out) - 1 == g["expected_accepted"]


@pytest.mark.parametrize("k,m", [(3, 0), (3, 3), (15, 0), (15, 3), (15, 7), (15, 15)])
def test_greedy_chain_planted_lengths(k, m):
    argmax, drafts = chain_greedy_case(100 + m, k, m)
    out = accept_greedy_chain(argmax, drafts)
    assert len(out) == m + 1 and 1 <= len(out) <= k + 1
    assert out[:m] == list(drafts[:m]) and out[m] == int(argmax[m])


def all_root_paths(parent):
    n = len(parent)
    paths = []
    for j in range(n):
        p, node = [], j
        while node >= 0:
            p.append(node)
            node = int(parent[node])
        paths.append(p[::-1])
    return paths


def brute_force_tree(argmax, tokens, parent):
    best = []
    for path in all_root_paths(parent):
        rows = [0] + [j + 1 for j in path[:-1]]
        if all(int(tokens[j]) == int(argmax[r]) for j, r in zip(path, rows)):
            if len(path) > len(best) or (len(path) == len(best) and path[-1] < best[-1]):
                best = path
    last_row = 0 if not best else best[-1] + 1
    return [int(tokens[j]) for j in best] + [int(argmax[last_row])]


@pytest.mark.parametrize("branch,length", [(0, 8), (1, 5), (2, 3), (-1, 0), (1, 1), (2, 8)])
def test_tree_planted(branch, length):
    parent, tokens, argmax = tree_greedy_case(300 + 7 * branch + length, 3, 8, branch, length)
    out = accept_greedy_tree(argmax, tokens, parent)
    assert out == brute_force_tree(argmax, tokens, parent)
    assert len(out) == length + 1


def test_tree_random_small_vocab_against_brute_force():
    rng = np.random.default_rng(9)
    for _ in range(300):
        n = int(rng.integers(1, 12))
        parent = np.array([-1 if j == 0 else int(rng.integers(-1, j)) for j in range(n)], dtype=np.int32)
        tokens = rng.integers(0, 3, n).astype(np.int32)
        argmax = rng.integers(0, 3, n + 1).astype(np.int32)
        assert accept_greedy_tree(argmax, tokens, parent) == brute_force_tree(argmax, tokens, parent)


def test_tree_chain_equals_greedy_chain():
    rng = np.random.default_rng(5)
    for _ in range(100):
        k = int(rng.integers(1, 16))
        drafts = rng.integers(0, 3, k).astype(np.int32)
        argmax = rng.integers(0, 3, k + 1).astype(np.int32)
        parent = np.arange(-1, k - 1, dtype=np.int32)
        assert accept_greedy_tree(argmax, drafts, parent) == accept_greedy_chain(argmax, drafts)


def dist(ids, probs):
    return (np.array(ids, dtype=np.int32), np.array(probs, dtype=np.float32))


def test_sampled_at_least_one_token_and_bonus_only_after_full_accept():
    rng = np.random.default_rng(2)
    for _ in range(500):
        k = int(rng.integers(1, 6))
        rows = []
        for _ in range(k + 1):
            ids = rng.permutation(6)[: int(rng.integers(1, 6))]
            w = rng.random(len(ids)) + 0.01
            rows.append(dist(ids, (w / w.sum()).astype(np.float32)))
        qrows = []
        for _ in range(k):
            ids = rng.permutation(6)[: int(rng.integers(1, 6))]
            w = rng.random(len(ids)) + 0.01
            qrows.append(dist(ids, (w / w.sum()).astype(np.float32)))
        drafts = [int(q[0][draw(q[1], rng.random())]) for q in qrows]
        u = rng.random((k + 1, 2)).astype(np.float32)
        out = accept_sampled(rows, qrows, drafts, u)
        assert 1 <= len(out) <= k + 1
        assert out[:-1] == drafts[: len(out) - 1]


def test_crafted_uniforms_force_accept_and_reject():
    p = dist([1, 2, 3], [0.5, 0.3, 0.2])
    q = dist([1, 2, 3], [0.2, 0.6, 0.2])
    bonus = dist([7], [1.0])
    # u = 0 accepts whenever p(x) > 0
    assert accept_sampled([p, bonus], [q], [2], [[0.0, 0.0], [0.0, 0.0]]) == [2, 7]
    # u = 1 - 2^-24 rejects when p(x) < q(x); the residual (p - q)+ is {1: .3} only
    assert accept_sampled([p, bonus], [q], [2], [[1 - 2**-24, 0.9], [0, 0]]) == [1]
    # a draft outside p's support is always rejected
    assert accept_sampled([p, bonus], [dist([9], [1.0])], [9], [[0.0, 0.0], [0, 0]]) == [1]
    # p == q: never rejected; zero residual falls back to p
    assert accept_sampled([p, bonus], [p], [3], [[1 - 2**-24, 0.0], [0, 0]]) == [3, 7]


def enumerate_emitted(p, q, grid):
    """P(first emitted token) by exact enumeration over drafts and a uniform grid."""
    ids_q, probs_q = q
    prob = {}
    weight = 1.0 / (len(grid) * len(grid))
    bonus = dist([-1], [1.0])
    for x, qx in zip(ids_q, probs_q):
        for u0 in grid:
            for u1 in grid:
                t = accept_sampled([p, bonus], [q], [int(x)], [[u0, u1], [0.0, 0.0]])[0]
                prob[t] = prob.get(t, 0.0) + float(qx) * weight
    return prob


def test_exact_enumeration_dyadic():
    # acceptance ratios 1, 1/2, 1, 0 (token 4 is outside p); residual
    # (3/8, 0, 0, 1/8) over p's support, CDF boundary 3/4: all multiples of 1/32
    p = dist([0, 1, 2, 3], [0.5, 0.25, 0.125, 0.125])
    q = dist([0, 1, 2, 4], [0.125, 0.5, 0.125, 0.25])
    grid = np.arange(32) / 32
    prob = enumerate_emitted(p, q, grid)
    assert prob == {0: 0.5, 1: 0.25, 2: 0.125, 3: 0.125}


def test_point_mass_draft_closed_form():
    # q = delta(c): accept with probability p(c), else draw from p without c
    p = dist([0, 1, 2, 3], [0.5, 0.25, 0.125, 0.125])
    bonus = dist([-1], [1.0])
    q = dist([1], [1.0])
    grid = np.arange(64) / 64
    accepted = [len(accept_sampled([p, bonus], [q], [1], [[u, 0.0], [0, 0]])) == 2 for u in grid]
    assert np.mean(accepted) == 0.25
    # on rejection the replacement never equals c and follows p without c: (2/3, 0, 1/6, 1/6)
    reps = [accept_sampled([p, bonus], [q], [1], [[0.999, u], [0, 0]])[0] for u in grid]
    counts = np.bincount(reps, minlength=4) / len(grid)
    assert counts[1] == 0.0
    np.testing.assert_allclose(counts, [2 / 3, 0, 1 / 6, 1 / 6], atol=1 / 64)
    # with c = 0 every boundary is dyadic and the enumeration gives p exactly
    q0 = dist([0], [1.0])
    assert enumerate_emitted(p, q0, np.arange(32) / 32) == {0: 0.5, 1: 0.25, 2: 0.125, 3: 0.125}


# ---------------------------------------------------------------- chi-square


CFG = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)


def make_case(rho, seed, k=3, vocab=4096):
    """Fixed p rows (k+1) and q rows (k) over `vocab`, policy applied to the top-64 pool."""
    from oracle.topk import topk_rows

    pl = logits(seed, (k + 1, vocab))
    if rho == "point":
        q_rows = None
    else:
        ql = correlated_logits(pl[:k], rho, seed + 1)
        qv, qi = topk_rows(ql, 64)
        q_rows = [policy_row(qv[i], qi[i], **CFG) for i in range(k)]
    pv, pi = topk_rows(pl, 64)
    p_rows = [policy_row(pv[i], pi[i], **CFG) for i in range(k + 1)]
    if q_rows is None:  # point-mass drafts: the second most likely target token
        q_rows = [dist([int(p_rows[i][0][1])], [1.0]) for i in range(k)]
    return p_rows, q_rows


def run_trials(p_rows, q_rows, n, seed):
    k = len(q_rows)
    ud = uniforms(seed, (n, k))
    u = uniforms(seed + 1, (n, k + 1, 2))
    out = []
    for b in range(n):
        drafts = [int(q_rows[i][0][draw(q_rows[i][1], ud[b, i])]) for i in range(k)]
        out.append(accept_sampled(p_rows, q_rows, drafts, u[b]))
    return out


def row_pvalues(p_rows, outs):
    pv = []
    for i in range(len(p_rows)):
        toks = [o[i] for o in outs if len(o) > i]
        pv.append(chi2_pvalue(toks, *p_rows[i]) if len(toks) >= 200 else 1.0)
    return pv


TRIALS = 200_000


@pytest.mark.parametrize("rho", [0.9, 0.0, 1.0, "point"])
def test_chi_square_emitted_tokens_follow_p(rho):
    p_rows, q_rows = make_case(rho, 1100 + (7 if rho == "point" else int(float(rho) * 10)))
    outs = run_trials(p_rows, q_rows, TRIALS, 42)
    pv = row_pvalues(p_rows, outs)
    assert min(pv) >= 1e-3, pv
    if rho == 1.0:  # q == p: every draft accepted
        assert all(len(o) == len(q_rows) + 1 for o in outs)


@pytest.mark.parametrize("rho", [0.9, "point"])
def test_chi_square_control_replacement_from_p_fails(rho, monkeypatch):
    p_rows, q_rows = make_case(rho, 1100 + (7 if rho == "point" else int(float(rho) * 10)))
    monkeypatch.setattr(acc, "residual_weights", lambda p, q: [float(x) for x in p[1]])
    outs = run_trials(p_rows, q_rows, TRIALS, 42)
    pv = row_pvalues(p_rows, outs)
    assert pv[0] < 1e-6, pv


# ------------------------------------------------- deterministic drafts


def test_point_mass_rule_equals_sampled_rule_with_delta_q():
    """The point-mass rule ([SD] §06) is the sampled rule with q = delta(d):
    two formulations, one through the residual (p - q)+, one removing d."""
    from oracle.accept import accept_point_mass

    for seed in range(6):
        p_rows, _ = make_case(0.9, 1300 + seed)
        g = np.random.default_rng(1310 + seed)
        for trial in range(300):
            drafts = []
            for i in range(3):
                ids = p_rows[i][0]
                drafts.append(int(ids[g.integers(len(ids))]) if g.random() < 0.8 else 4095 - i)
            u = uniforms(1320 + seed * 1000 + trial, (4, 2))
            q_rows = [dist([d], [1.0]) for d in drafts]
            assert accept_point_mass(p_rows, drafts, u) == accept_sampled(p_rows, q_rows, drafts, u)


def test_point_mass_rule_closed_form_grid():
    """Accept with probability p(c), else a draw from p without c; together
    the emitted token follows p exactly (dyadic boundaries, exact grid)."""
    from oracle.accept import accept_point_mass

    p = dist([0, 1, 2, 3], [0.5, 0.25, 0.125, 0.125])
    bonus = dist([9], [1.0])
    grid = np.arange(64) / 64
    accepted = [len(accept_point_mass([p, bonus], [0], [[u0, 0.0], [0, 0]])) == 2 for u0 in grid]
    assert np.mean(accepted) == 0.5
    reps = [accept_point_mass([p, bonus], [0], [[0.999, u1], [0, 0]])[0] for u1 in grid]
    assert list(np.bincount(reps, minlength=4) / len(grid)) == [0.0, 0.5, 0.25, 0.25]
    g32 = np.arange(32) / 32
    first = [accept_point_mass([p, bonus], [0], [[u0, u1], [0, 0]])[0] for u0 in g32 for u1 in g32]
    assert list(np.bincount(first, minlength=4) / len(first)) == [0.5, 0.25, 0.125, 0.125]


def test_naive_verify_closed_forms():
    """Naive-sampling verify ([PR] "Code map"): every emitted token is a draw
    from its row's p, so the first token follows p_0 exactly, and the window
    length is 1 + the number of leading rows whose draw equals the draft:
    P(n = 1) = 1 - p_0(d_0), P(n = 2) = p_0(d_0)(1 - p_1(d_1)),
    P(n = 3) = p_0(d_0) p_1(d_1)."""
    from oracle.accept import accept_naive

    p0 = dist([0, 1, 2, 3], [0.5, 0.25, 0.125, 0.125])
    p1 = dist([5, 6], [0.75, 0.25])
    p2 = dist([9], [1.0])
    grid = np.arange(32) / 32
    outs = [accept_naive([p0, p1, p2], [1, 5], [[0, a], [0, b], [0, 0.5]]) for a in grid for b in grid]
    n = len(outs)
    first = np.bincount([o[0] for o in outs], minlength=4) / n
    assert list(first) == [0.5, 0.25, 0.125, 0.125]
    lengths = np.bincount([len(o) for o in outs], minlength=4) / n
    assert list(lengths[1:]) == [0.75, 0.25 * 0.25, 0.25 * 0.75]
    second = [o[1] for o in outs if len(o) >= 2]
    assert second.count(5) / len(second) == 0.75
    assert all(o[-1] == 9 for o in outs if len(o) == 3)


def test_naive_verify_on_one_hot_rows_is_greedy():
    from oracle.accept import accept_naive

    g = np.random.default_rng(1330)
    for trial in range(200):
        k = int(g.integers(0, 8))
        argmax = g.integers(0, 50, size=k + 1)
        drafts = np.where(g.random(k) < 0.7, argmax[:k], g.integers(0, 50, size=k))
        rows = [dist([int(a)], [1.0]) for a in argmax]
        u = uniforms(1331 + trial, (k + 1, 2))
        assert accept_naive(rows, drafts, u) == accept_greedy_chain(argmax, drafts)


def run_naive_trials(p_rows, q_rows, n, seed):
    from oracle.accept import accept_naive

    k = len(q_rows)
    ud = uniforms(seed, (n, k))
    u = uniforms(seed + 1, (n, k + 1, 2))
    out = []
    for b in range(n):
        drafts = [int(q_rows[i][0][draw(q_rows[i][1], ud[b, i])]) for i in range(k)]
        out.append(accept_naive(p_rows, drafts, u[b]))
    return out


def test_chi_square_naive_verify_follows_p():
    p_rows, q_rows = make_case(0.9, 1109)
    outs = run_naive_trials(p_rows, q_rows, TRIALS, 43)
    pv = row_pvalues(p_rows, outs)
    assert min(pv) >= 1e-3, pv


def test_chi_square_control_naive_greedy_draw_fails(monkeypatch):
    """Planted mistake: each row emits its most likely token instead of a draw."""
    p_rows, q_rows = make_case(0.9, 1109)
    monkeypatch.setattr(acc, "draw", lambda probs, u: 0)
    outs = run_naive_trials(p_rows, q_rows, TRIALS, 43)
    pv = row_pvalues(p_rows, outs)
    assert pv[0] < 1e-6, pv


# --------------------------------------------- naive verify of a token tree


def test_naive_tree_walk_on_a_chain_is_the_chain_rule():
    from oracle.accept import accept_naive, accept_naive_tree

    for seed in range(4):
        p_rows, _ = make_case(0.9, 1400 + seed)
        g = np.random.default_rng(1410 + seed)
        for trial in range(300):
            drafts = [int(p_rows[i][0][g.integers(len(p_rows[i][0]))]) for i in range(3)]
            u = uniforms(1420 + seed * 1000 + trial, (4, 2))
            assert accept_naive_tree(p_rows, drafts, [-1, 0, 1], u) == accept_naive(p_rows, drafts, u)


def test_naive_tree_walk_exact_enumeration():
    """Root draw follows p_0 exactly; the walk enters the child carrying the
    draw and continues with that child's row (dyadic grid, exact)."""
    from oracle.accept import accept_naive_tree

    p0 = dist([0, 1, 2, 3], [0.5, 0.25, 0.125, 0.125])
    p_a = dist([5, 6], [0.75, 0.25])      # row of node 0 (token 1)
    p_b = dist([7, 8], [0.5, 0.5])        # row of node 1 (token 2)
    p_c = dist([9], [1.0])                # row of node 2 (token 5, child of node 0)
    tokens, parent = [1, 2, 5], [-1, -1, 0]
    grid = np.arange(32) / 32
    outs = [accept_naive_tree([p0, p_a, p_b, p_c], tokens, parent, [[0, a], [0, b], [0, c], [0, 0.5]])
            for a in grid for b in grid for c in (0.25, 0.75)]
    n = len(outs)
    assert list(np.bincount([o[0] for o in outs], minlength=4) / n) == [0.5, 0.25, 0.125, 0.125]
    via_a = [o for o in outs if o[0] == 1]
    assert all(len(o) >= 2 for o in via_a) and sum(o[1] == 5 for o in via_a) / len(via_a) == 0.75
    assert all(o == [1, 5, 9] for o in via_a if o[1] == 5)
    via_b = [o for o in outs if o[0] == 2]
    assert all(len(o) == 2 and o[1] in (7, 8) for o in via_b)
    assert all(len(o) == 1 for o in outs if o[0] in (0, 3))


def test_naive_tree_walk_on_one_hot_rows_is_the_greedy_tree_walk():
    from oracle.accept import accept_naive_tree
    from oracle.lookup import lookup_tree

    g = np.random.default_rng(1430)
    for trial in range(300):
        ctx = list(g.integers(0, 6, size=int(g.integers(10, 120))))
        tokens, parent = lookup_tree(ctx, 2, 3, 5, 16)      # a trie: siblings differ
        if not tokens:
            continue
        am = g.integers(0, 6, size=len(tokens) + 1)
        rows = [dist([int(a)], [1.0]) for a in am]
        u = uniforms(1431 + trial, (len(tokens) + 1, 2))
        assert accept_naive_tree(rows, tokens, parent, u) == accept_greedy_tree(am, tokens, parent)


def tree_rows_case(seed, n_nodes=24):
    """A random trie of n_nodes (3 branches) and its n_nodes + 1 policy rows."""
    from oracle.topk import topk_rows

    g = np.random.default_rng(seed)
    pl = logits(seed, (n_nodes + 1, 4096))
    pv, pi = topk_rows(pl, 64)
    rows = [policy_row(pv[i], pi[i], **CFG) for i in range(n_nodes + 1)]
    tokens, parent = [], []
    # children tokens drawn from the parent row's support, so the walk goes deep
    while len(tokens) < n_nodes:
        node = int(g.integers(-1, len(tokens)))
        prow = 0 if node < 0 else node + 1
        sib = {tokens[j] for j in range(len(tokens)) if parent[j] == node}
        cand = [int(t) for t in rows[prow][0][:4] if int(t) not in sib]
        if cand:
            tokens.append(cand[0])
            parent.append(node)
    return rows, tokens, parent


def naive_tree_row_draws(rows, tokens, parent, outs):
    """Per row, the tokens drawn there: the emitted token at each step of each walk."""
    per = [[] for _ in rows]
    for o in outs:
        node, row = -1, 0
        for x in o:
            per[row].append(x)
            child = next((j for j in range(len(tokens)) if parent[j] == node and tokens[j] == x), None)
            if child is None:
                break
            node, row = child, child + 1
    return per


def naive_tree_pvalues(seed):
    from oracle.accept import accept_naive_tree

    rows, tokens, parent = tree_rows_case(seed)
    u = uniforms(seed + 1, (TRIALS, len(tokens) + 1, 2))
    outs = [accept_naive_tree(rows, tokens, parent, u[b]) for b in range(TRIALS)]
    per = naive_tree_row_draws(rows, tokens, parent, outs)
    return [chi2_pvalue(d, *rows[r]) for r, d in enumerate(per) if len(d) >= 200]


def test_chi_square_naive_tree_walk_follows_p():
    """Every visited row's draws follow its p: one test per row (25 rows), so
    the threshold is family-wise, 1e-3 over the number of rows (Bonferroni)."""
    pv = naive_tree_pvalues(1440)
    assert len(pv) >= 3 and min(pv) >= 1e-3 / len(pv), pv


def test_chi_square_control_naive_tree_greedy_draw_fails(monkeypatch):
    """Planted mistake: every row emits its most likely token instead of a draw."""
    monkeypatch.setattr(acc, "draw", lambda probs, u: 0)
    pv = naive_tree_pvalues(1440)
    assert pv[0] < 1e-6, pv
