"""GPU parity of spec_accept_rows.

Sampled windows follow section 03 of "Speculative decoding on RDNA": tokens
and counts must equal the oracle's under the same uniforms (both decide in
fp64 from the same fp32 probabilities, so no near-tie exception is needed
here), and the GPU's emitted tokens must pass the 200,000-trial chi-square
test against p.  Greedy chains and trees use planted accept lengths.
"""

import numpy as np
import pytest
import torch

import verify_sampling_amd as vs
from gpu_common import dev, host
from oracle.accept import accept_greedy_chain, accept_greedy_tree, accept_sampled
from oracle.policy import draw, policy_row
from oracle.topk import topk_rows
from stats import chi2_pvalue
from synth import (VOCAB, chain_greedy_case, correlated_logits, logits, tree_greedy_case,
                   uniforms)

pytestmark = pytest.mark.gpu
CFG = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)
W = 64


def pack(rows, width=W):
    n = len(rows)
    ids = np.full((n, width), -1, dtype=np.int32)
    probs = np.zeros((n, width), dtype=np.float32)
    lens = np.zeros(n, dtype=np.int32)
    for i, (t, p) in enumerate(rows):
        ids[i, :len(t)] = t
        probs[i, :len(p)] = p
        lens[i] = len(t)
    return ids, probs, lens


def make_case(rho, seed, k=3, vocab=4096):
    pl = logits(seed, (k + 1, vocab))
    pv, pi = topk_rows(pl, 64)
    p_rows = [policy_row(pv[i], pi[i], **CFG) for i in range(k + 1)]
    if rho == "point":
        q_rows = [(np.array([p_rows[i][0][1]], dtype=np.int32), np.array([1.0], dtype=np.float32))
                  for i in range(k)]
    else:
        ql = correlated_logits(pl[:k], rho, seed + 1)
        qv, qi = topk_rows(ql, 64)
        q_rows = [policy_row(qv[i], qi[i], **CFG) for i in range(k)]
    return p_rows, q_rows


TRIALS = 200_000


@pytest.mark.parametrize("rho", [0.9, 0.0, 1.0, "point"])
def test_sampled_windows_match_oracle_and_follow_p(rho):
    k = 3
    p_rows, q_rows = make_case(rho, 1800 + (7 if rho == "point" else int(float(rho) * 10)))
    ud = uniforms(1810, (TRIALS, k))
    u = uniforms(1811, (TRIALS, k + 1, 2))
    drafts = np.array([[int(q_rows[i][0][draw(q_rows[i][1], ud[b, i])]) for i in range(k)]
                       for b in range(TRIALS)], dtype=np.int32)
    pi, pp, pln = pack(p_rows)
    qi, qp, qln = pack(q_rows)
    tok, n = vs.spec_accept_rows(vs.ACCEPT_SAMPLED, dev(drafts), (dev(pi), dev(pp), dev(pln)),
                                 (dev(qi), dev(qp), dev(qln)), u=dev(u), p_win_stride=0,
                                 q_win_stride=0)
    tok, n = host(tok), host(n)
    mism = 0
    for b in range(TRIALS):
        want = accept_sampled(p_rows, q_rows, drafts[b], u[b])
        got = list(tok[b, :n[b]])
        if got != want or (tok[b, n[b]:] != -1).any():
            mism += 1
    assert mism == 0, f"{mism} windows differ"
    for i in range(k + 1):
        toks = tok[n > i, i]
        if len(toks) >= 200:
            assert chi2_pvalue(toks, *p_rows[i]) >= 1e-3, i


@pytest.mark.parametrize("m", [0, 3, 7, 15])
def test_greedy_chain_planted(m):
    k = 15
    argmax, drafts = chain_greedy_case(1820 + m, k, m)
    p_ids = np.full((k + 1, 4), -1, dtype=np.int32)
    p_ids[:, 0] = argmax
    tok, n = vs.spec_accept_rows(vs.ACCEPT_GREEDY, dev(drafts[None, :]), (dev(p_ids), None, None))
    tok, n = host(tok), host(n)
    assert list(tok[0, :n[0]]) == accept_greedy_chain(argmax, drafts)
    assert n[0] == m + 1 and (tok[0, n[0]:] == -1).all()


def test_tree_planted_batch():
    cases = [(0, 8), (1, 5), (2, 3), (-1, 0), (1, 1), (2, 8), (0, 2), (1, 8)]
    B, n_nodes = len(cases), 24
    parents = np.zeros((B, n_nodes), dtype=np.int32)
    tokens = np.zeros((B, n_nodes), dtype=np.int32)
    p_ids = np.full((B * (n_nodes + 1), 2), -1, dtype=np.int32)
    want = []
    for b, (br, ln) in enumerate(cases):
        par, tk, am = tree_greedy_case(1830 + b, 3, 8, br, ln)
        parents[b], tokens[b] = par, tk
        p_ids[b * (n_nodes + 1):(b + 1) * (n_nodes + 1), 0] = am
        want.append(accept_greedy_tree(am, tk, par))
    tok, n = vs.spec_accept_rows(vs.ACCEPT_GREEDY_TREE, dev(tokens), (dev(p_ids), None, None),
                                 parent=dev(parents))
    tok, n = host(tok), host(n)
    for b in range(B):
        assert list(tok[b, :n[b]]) == want[b], b
        assert n[b] == cases[b][1] + 1


def test_tree_random_small_vocab():
    g = np.random.default_rng(1840)
    B, k = 2000, 12
    parents = np.array([[-1 if j == 0 else int(g.integers(-1, j)) for j in range(k)]
                        for _ in range(B)], dtype=np.int32)
    tokens = g.integers(0, 3, (B, k)).astype(np.int32)
    am = g.integers(0, 3, (B, k + 1)).astype(np.int32)
    p_ids = am.reshape(-1, 1).copy()
    tok, n = vs.spec_accept_rows(vs.ACCEPT_GREEDY_TREE, dev(tokens), (dev(p_ids), None, None),
                                 parent=dev(parents))
    tok, n = host(tok), host(n)
    for b in range(B):
        assert list(tok[b, :n[b]]) == accept_greedy_tree(am[b], tokens[b], parents[b]), b


def test_greedy_random_chains_and_k0():
    g = np.random.default_rng(1841)
    B, k = 3000, 5
    drafts = g.integers(0, 2, (B, k)).astype(np.int32)
    am = g.integers(0, 2, (B, k + 1)).astype(np.int32)
    tok, n = vs.spec_accept_rows(vs.ACCEPT_GREEDY, dev(drafts), (dev(am.reshape(-1, 1).copy()), None, None))
    tok, n = host(tok), host(n)
    for b in range(B):
        assert list(tok[b, :n[b]]) == accept_greedy_chain(am[b], drafts[b])
    # k = 0: the window is one plain decode step
    d0 = torch.zeros((4, 0), dtype=torch.int32, device="cuda:0")
    am0 = np.array([[5], [6], [7], [8]], dtype=np.int32)
    tok, n = vs.spec_accept_rows(vs.ACCEPT_GREEDY, d0, (dev(am0), None, None))
    assert list(host(n)) == [1, 1, 1, 1] and list(host(tok)[:, 0]) == [5, 6, 7, 8]


def test_sampled_per_window_distributions():
    """Distinct p and q rows per window (stride k+1 and k), k = 5, random supports."""
    g = np.random.default_rng(1842)
    B, k = 3000, 5
    p_rows_all, q_rows_all = [], []
    for _ in range(B * (k + 1)):
        t = g.permutation(10)[: int(g.integers(1, 8))].astype(np.int32)
        w = g.random(len(t)) + 0.01
        p_rows_all.append((t, (w / w.sum()).astype(np.float32)))
    for _ in range(B * k):
        t = g.permutation(10)[: int(g.integers(1, 8))].astype(np.int32)
        w = g.random(len(t)) + 0.01
        q_rows_all.append((t, (w / w.sum()).astype(np.float32)))
    drafts = np.array([[int(q_rows_all[b * k + i][0][draw(q_rows_all[b * k + i][1], g.random())])
                        for i in range(k)] for b in range(B)], dtype=np.int32)
    u = g.random((B, k + 1, 2)).astype(np.float32)
    pi, pp, pln = pack(p_rows_all, 8)
    qi, qp, qln = pack(q_rows_all, 8)
    tok, n = vs.spec_accept_rows(vs.ACCEPT_SAMPLED, dev(drafts), (dev(pi), dev(pp), dev(pln)),
                                 (dev(qi), dev(qp), dev(qln)), u=dev(u))
    tok, n = host(tok), host(n)
    for b in range(B):
        want = accept_sampled(p_rows_all[b * (k + 1):(b + 1) * (k + 1)],
                              q_rows_all[b * k:(b + 1) * k], drafts[b], u[b])
        assert list(tok[b, :n[b]]) == want, b


def deterministic_drafts(p_rows, n, seed, k=3):
    """Per window: row i's draft is a token of p_i's support (80%) or one outside it."""
    g = np.random.default_rng(seed)
    out = np.empty((n, k), dtype=np.int32)
    for i in range(k):
        ids = p_rows[i][0]
        pick = ids[g.integers(0, len(ids), size=n)]
        out[:, i] = np.where(g.random(n) < 0.8, pick, 4095 - i)
    return out


@pytest.mark.parametrize("mode", ["point", "naive"])
def test_deterministic_draft_modes_match_oracle_and_follow_p(mode):
    """Point-mass rule ([SD] §06) and naive-sampling verify ([PR] "Code map")
    on 200,000 windows: tokens and counts equal the oracle's under the same
    uniforms, and every row's emitted tokens pass the chi-square test against
    p.  The point-mass mode also equals the sampled mode with q = delta(d)."""
    from oracle.accept import accept_naive, accept_point_mass

    k = 3
    p_rows, _ = make_case(0.9, 1850)
    drafts = deterministic_drafts(p_rows, TRIALS, 1851)
    u = uniforms(1852, (TRIALS, k + 1, 2))
    pi, pp, pln = pack(p_rows)
    m = vs.ACCEPT_POINT_MASS if mode == "point" else vs.ACCEPT_NAIVE
    tok, n = vs.spec_accept_rows(m, dev(drafts), (dev(pi), dev(pp), dev(pln)), u=dev(u),
                                 p_win_stride=0)
    tok, n = host(tok), host(n)
    ref = accept_point_mass if mode == "point" else accept_naive
    mism = 0
    for b in range(TRIALS):
        got = list(tok[b, :n[b]])
        if got != ref(p_rows, drafts[b], u[b]) or (tok[b, n[b]:] != -1).any():
            mism += 1
    assert mism == 0, f"{mism} windows differ"
    for i in range(k + 1):
        toks = tok[n > i, i]
        if len(toks) >= 200:
            assert chi2_pvalue(toks, *p_rows[i]) >= 1e-3, i
    if mode == "point":
        q = np.full((TRIALS * k, 1), -1, dtype=np.int32)
        q[:, 0] = drafts.reshape(-1)
        qp = np.ones((TRIALS * k, 1), dtype=np.float32)
        ql = np.ones(TRIALS * k, dtype=np.int32)
        tok2, n2 = vs.spec_accept_rows(vs.ACCEPT_SAMPLED, dev(drafts), (dev(pi), dev(pp), dev(pln)),
                                       (dev(q), dev(qp), dev(ql)), u=dev(u), p_win_stride=0)
        assert np.array_equal(host(tok2), tok) and np.array_equal(host(n2), n)


def test_prompt_lookup_trees_greedy_walk():
    """Token trees drafted by prompt lookup (vs_lookup_tree: top 3 matches of
    the last 3 tokens, depth 8, 24 nodes) over a context of copied lines,
    verified by the greedy tree walk.  The target's argmax rows follow what
    the context really does next: the root row and every node whose path is
    a prefix of the true continuation predict its next token, other rows a
    token of their own.  Trees shorter than 24 nodes are padded with nodes
    that never agree (token -2).  Every drafted tree equals the oracle
    drafter's (oracle.lookup) and the GPU tokens equal the oracle's."""
    from oracle.lookup import lookup_tree
    from synth import lookup_context

    ctx = lookup_context(1870, 40000)
    g = np.random.default_rng(1871)
    B, K = 512, 24
    tokens = np.full((B, K), -2, dtype=np.int32)
    parents = np.full((B, K), -1, dtype=np.int32)
    p_ids = np.full((B * (K + 1), 2), -1, dtype=np.int32)
    want, sizes = [], []
    for b in range(B):
        e = int(g.integers(1000, len(ctx) - 16))
        tk, par = vs.lookup_tree(ctx[:e], 3, 3, 8, K)
        want_t, want_p = lookup_tree(list(ctx[:e]), 3, 3, 8, K)
        assert list(tk) == want_t and list(par) == want_p, b
        truth = ctx[e:e + 10]
        sizes.append(len(tk))
        tokens[b, :len(tk)], parents[b, :len(tk)] = tk, par
        am = np.empty(K + 1, dtype=np.int32)
        am[0] = truth[0]
        for j in range(K):
            path, q = [], j
            while q >= 0 and j < len(tk):
                path.append(int(tokens[b, q]))
                q = int(parents[b, q])
            path.reverse()
            d = len(path)
            on_truth = j < len(tk) and list(truth[:d]) == path
            am[j + 1] = truth[d] if on_truth else int(g.integers(0, VOCAB))
        p_ids[b * (K + 1):(b + 1) * (K + 1), 0] = am
        want.append(accept_greedy_tree(am, tokens[b], parents[b]))
    tok, n = vs.spec_accept_rows(vs.ACCEPT_GREEDY_TREE, dev(tokens), (dev(p_ids), None, None),
                                 parent=dev(parents))
    tok, n = host(tok), host(n)
    for b in range(B):
        assert list(tok[b, :n[b]]) == want[b], b
    print(f"mean tree nodes {np.mean(sizes):.1f}; mean emitted per window {np.mean(n):.2f}")
    assert np.mean(n) > 1.5   # the trees do contain the context's next tokens


def test_naive_tree_walk_matches_oracle_and_follows_p():
    """Naive-sampling verify of a 24-node token tree over 200,000 windows
    (one tree and its 25 rows shared by all windows, fresh uniforms per
    window): tokens and counts equal the oracle's, and every row's draws
    pass the chi-square test against its p (family-wise 1e-3 over the rows
    tested)."""
    from oracle.accept import accept_naive_tree
    import test_oracle_accept as toa

    rows, tokens, parent = toa.tree_rows_case(1860)
    K = len(tokens)
    u = uniforms(1861, (TRIALS, K + 1, 2))
    pi, pp, pln = pack(rows)
    tk = np.broadcast_to(np.array(tokens, dtype=np.int32), (TRIALS, K)).copy()
    pr = np.broadcast_to(np.array(parent, dtype=np.int32), (TRIALS, K)).copy()
    tok, n = vs.spec_accept_rows(vs.ACCEPT_NAIVE_TREE, dev(tk), (dev(pi), dev(pp), dev(pln)),
                                 u=dev(u), parent=dev(pr), p_win_stride=0)
    tok, n = host(tok), host(n)
    outs = []
    mism = 0
    for b in range(TRIALS):
        got = list(tok[b, :n[b]])
        outs.append(got)
        if got != accept_naive_tree(rows, tokens, parent, u[b]) or (tok[b, n[b]:] != -1).any():
            mism += 1
    assert mism == 0, f"{mism} windows differ"
    per = toa.naive_tree_row_draws(rows, tokens, parent, outs)
    pv = [chi2_pvalue(d, *rows[r]) for r, d in enumerate(per) if len(d) >= 200]
    assert len(pv) >= 3 and min(pv) >= 1e-3 / len(pv), pv


def test_naive_tree_walk_on_drafted_trees():
    """Prompt-lookup trees (a different tree per window, padded with
    never-matching nodes, one malformed parent) with seeded per-window rows
    that favour the tree's tokens, fed identically to both sides: GPU
    tokens equal the oracle's."""
    from oracle.accept import accept_naive_tree
    from synth import lookup_context

    ctx = lookup_context(1870, 20000, vocab=4096)
    g = np.random.default_rng(1872)
    B, K = 256, 24
    tokens = np.full((B, K), -2, dtype=np.int32)
    parents = np.full((B, K), -1, dtype=np.int32)
    rows = []
    for b in range(B):
        e = int(g.integers(1000, len(ctx) - 16))
        tk, par = vs.lookup_tree(ctx[:e], 3, 3, 8, K)
        tokens[b, :len(tk)], parents[b, :len(tk)] = tk, par
        for r in range(K + 1):
            # row r: its children's tokens plus random ones, children weighted up
            kids = [int(tk[j]) for j in range(len(tk)) if (par[j] + 1 if par[j] >= 0 else 0) == r]
            other = [int(t) for t in g.integers(0, 4096, size=12) if int(t) not in kids]
            ids = np.array(kids + other, dtype=np.int32)
            w = np.concatenate([np.full(len(kids), 16.0), g.random(len(other))])
            rows.append((ids, (w / w.sum()).astype(np.float32)))
    parents[0, K - 1] = K + 3                         # malformed: never reached
    pi, pp, pln = pack(rows)
    u = uniforms(1874, (B, K + 1, 2))
    tok, n = vs.spec_accept_rows(vs.ACCEPT_NAIVE_TREE, dev(tokens), (dev(pi), dev(pp), dev(pln)),
                                 u=dev(u), parent=dev(parents))
    tok, n = host(tok), host(n)
    for b in range(B):
        want = accept_naive_tree(rows[b * (K + 1):(b + 1) * (K + 1)], tokens[b], parents[b], u[b])
        assert list(tok[b, :n[b]]) == want, b
    print(f"mean emitted per window {np.mean(n):.2f}")
    assert np.mean(n) > 1.5


def test_maximum_depth_every_mode():
    """k = 63 drafts, the most a window takes (64 rows), in every mode.  Some
    windows accept every draft and the bonus row, others stop at a planted
    position; tokens and counts equal the oracle's."""
    from oracle.accept import accept_naive, accept_naive_tree, accept_point_mass

    g = np.random.default_rng(1880)
    B, k = 128, 63

    # greedy chain: window b disagrees first at draft b (b = 63 and above: never)
    am = g.integers(0, 50, (B, k + 1)).astype(np.int32)
    drafts = am[:, :k].copy()
    for b in range(min(B, k)):
        drafts[b, b] = am[b, b] + 1
    tok, n = vs.spec_accept_rows(vs.ACCEPT_GREEDY, dev(drafts),
                                 (dev(am.reshape(-1, 1).copy()), None, None))
    tok, n = host(tok), host(n)
    for b in range(B):
        assert list(tok[b, :n[b]]) == accept_greedy_chain(am[b], drafts[b]), b
        assert n[b] == min(b, k) + 1
    assert (tok[k:, :] == am[k:, :]).all()  # all 63 drafts and the bonus

    # greedy tree: window 0 a 63-node path that agrees everywhere, the rest random
    parents = np.array([[-1 if j == 0 else int(g.integers(-1, j)) for j in range(k)]
                        for _ in range(B)], dtype=np.int32)
    parents[0] = np.arange(-1, k - 1)
    tokens = g.integers(0, 3, (B, k)).astype(np.int32)
    am = g.integers(0, 3, (B, k + 1)).astype(np.int32)
    tokens[0] = am[0, :k]
    tok, n = vs.spec_accept_rows(vs.ACCEPT_GREEDY_TREE, dev(tokens),
                                 (dev(am.reshape(-1, 1).copy()), None, None), parent=dev(parents))
    tok, n = host(tok), host(n)
    for b in range(B):
        assert list(tok[b, :n[b]]) == accept_greedy_tree(am[b], tokens[b], parents[b]), b
    assert n[0] == k + 1

    # per-window p and q rows: even windows one-hot on a shared token (every
    # draft accepted), odd windows random supports over 10 tokens
    def row(b):
        if b % 2 == 0:
            t = np.array([int(g.integers(0, 10))], dtype=np.int32)
            return t, np.ones(1, dtype=np.float32)
        t = g.permutation(10)[: int(g.integers(1, 8))].astype(np.int32)
        w = g.random(len(t)) + 0.01
        return t, (w / w.sum()).astype(np.float32)

    p_rows = [row(b) for b in range(B) for _ in range(k + 1)]
    q_rows = [p_rows[b * (k + 1) + i] if b % 2 == 0 else row(b) for b in range(B) for i in range(k)]
    drafts = np.array([[int(q_rows[b * k + i][0][draw(q_rows[b * k + i][1], g.random())])
                        for i in range(k)] for b in range(B)], dtype=np.int32)
    u = g.random((B, k + 1, 2)).astype(np.float32)
    pi, pp, pln = pack(p_rows, 8)
    qi, qp, qln = pack(q_rows, 8)
    P = (dev(pi), dev(pp), dev(pln))
    tok, n = vs.spec_accept_rows(vs.ACCEPT_SAMPLED, dev(drafts), P, (dev(qi), dev(qp), dev(qln)),
                                 u=dev(u))
    tok, n = host(tok), host(n)
    for b in range(B):
        want = accept_sampled(p_rows[b * (k + 1):(b + 1) * (k + 1)], q_rows[b * k:(b + 1) * k],
                              drafts[b], u[b])
        assert list(tok[b, :n[b]]) == want, b
    assert (n[0::2] == k + 1).all()

    # deterministic drafts on the same p rows: point mass and naive sampling
    for mode, ref in ((vs.ACCEPT_POINT_MASS, accept_point_mass), (vs.ACCEPT_NAIVE, accept_naive)):
        tok, n = vs.spec_accept_rows(mode, dev(drafts), P, u=dev(u))
        tok, n = host(tok), host(n)
        for b in range(B):
            want = ref(p_rows[b * (k + 1):(b + 1) * (k + 1)], drafts[b], u[b])
            assert list(tok[b, :n[b]]) == want, (mode, b)
            assert (tok[b, n[b]:] == -1).all(), (mode, b)
        assert (n[0::2] == k + 1).all()

    # naive sampling down a 63-node tree, per-window rows; window 0 a path
    # whose one-hot rows agree with every node
    par = parents.copy()
    tk = np.array([[int(p_rows[b * (k + 1) + (par[b, j] + 1)][0][0]) for j in range(k)]
                   for b in range(B)], dtype=np.int32)
    tok, n = vs.spec_accept_rows(vs.ACCEPT_NAIVE_TREE, dev(tk), P, u=dev(u), parent=dev(par))
    tok, n = host(tok), host(n)
    for b in range(B):
        want = accept_naive_tree(p_rows[b * (k + 1):(b + 1) * (k + 1)], tk[b], par[b], u[b])
        assert list(tok[b, :n[b]]) == want, b
    assert n[0] == k + 1
