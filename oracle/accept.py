"""Acceptance of one speculative window.

Greedy chain: [SD] "Speculative decoding on RDNA", §02: accept the longest
prefix of drafts equal to the target's argmax; §01 (figure "one speculative
window" and the text under it): the window then emits the target's own
choice at the first disagreement, or a bonus token after the last row when
every draft is accepted, so it always emits at least one token.

Sampled chain: [SD] §03 "Sampled requests: rejection sampling", steps 1-4:
draft x ~ q; accept with probability min(1, p(x)/q(x)); on rejection emit
a draw from the residual (p - q)+ renormalised and end the window; if all
drafts are accepted, draw the bonus from p at the last row.  With a
point-mass draft q = delta(c) ([SD] §06) the same rule accepts with
probability p(c) and otherwise draws from p without c.

Deterministic drafts (the draft is a token, not a distribution):
  * point-mass rule, [SD] §06 (n-gram takeovers): the sampled rule with
    q = delta(d): accept d with probability p(d), otherwise emit a draw from
    p with d removed, renormalised;
  * naive-sampling verify, [PR] "Code map" (the generic chain's greedy and
    temp > 0 verify, exact for any deterministic draft): each verify row
    draws its own token from p and the window keeps going while that token
    equals the draft; the first differing draw is emitted and ends the
    window, and after k matches the bonus is drawn from the last row;
  * naive-sampling verify of a token tree (deterministic drafts, e.g. the
    prompt-lookup trees of [TREE]): start at the root row, draw from its p,
    emit the draw, and move to the child whose token it is (the
    lowest-numbered one if siblings repeat a token), continuing with that
    child's row; a draw that no child carries ends the window.  Every
    emitted token is a draw from its row's p, so the walk is lossless.

Greedy tree: [TREE] "Spend the budget on a tree, not a longer guess":
several continuations sharing a prefix are verified in one pass and the
longest branch the target agrees with is accepted.

Readings taken:
  * the accept test is u0 * q(x) < p(x) with u0 in [0, 1), evaluated in
    fp64 from fp32 probabilities (the product of two fp32 values is exact
    in fp64), which is acceptance with probability min(1, p/q);
  * p(x) and q(x) are the total probability the distribution gives token
    x; a token outside the support has probability 0, so a draft outside
    p's support is always rejected;
  * the residual is r_j = max(0, p_j - q(t_j)) over p's support in pool
    order, in fp64; if its total is 0 the replacement is drawn from p;
  * row i uses the uniforms u[i][0] (accept test) and u[i][1]
    (replacement or bonus draw); the bonus uses u[k][1].  The naive verify
    has no accept test: row i draws with u[i][1];
  * point-mass rule: u0 < p(d) (u0 * 1 in the sampled test); if p has no
    mass outside d the replacement is drawn from p, as for a zero residual;
  * a draw from an empty target row is -1 and always ends the window;
  * tree row r (0 = root, 1 + j = node j) draws with u[r][1]; a node whose
    parent lies outside [-1, j) is never reached;
  * a target row with an empty distribution emits token -1 (not a
    token; the policy only yields one when every candidate slot is empty);
  * argmax ties go to the lowest token id (the pool order), so a row's
    argmax is the first entry of its pool;
  * in a tree, row 0 is the root and row 1 + j is node j; the accepted
    branch is the longest agreeing one, the lowest-numbered end node on a
    tie.
"""

from __future__ import annotations

import numpy as np

from .policy import draw, draw_weights


def accept_greedy_chain(target_argmax, drafts) -> list[int]:
    out = []
    k = len(drafts)
    for i in range(k):
        d = int(drafts[i])
        if d == int(target_argmax[i]):
            out.append(d)
        else:
            out.append(int(target_argmax[i]))
            return out
    out.append(int(target_argmax[k]))
    return out


def accept_greedy_tree(target_argmax, tokens, parent) -> list[int]:
    """target_argmax [n+1] (row 0 = root), tokens [n], parent [n] (-1 = root).

    A node agrees with the target when its token equals the argmax of its
    parent's row and its parent agrees (the root always does).  The
    accepted branch ends at the deepest agreeing node (lowest node number
    on a tie); the window emits that branch's tokens, then the argmax of
    its last row.  ``parent[j] < j`` is required.
    """
    n = len(tokens)
    agrees = [False] * n
    depth = [0] * n
    for j in range(n):
        pj = int(parent[j])
        parent_row = 0 if pj < 0 else pj + 1
        parent_ok = True if pj < 0 else agrees[pj]
        agrees[j] = parent_ok and int(tokens[j]) == int(target_argmax[parent_row])
        depth[j] = 1 if pj < 0 else depth[pj] + 1
    best = -1
    for j in range(n):
        if agrees[j] and (best < 0 or depth[j] > depth[best]):
            best = j
    path = []
    j = best
    while j >= 0:
        path.append(j)
        j = int(parent[j])
    path.reverse()
    out = [int(tokens[j]) for j in path]
    out.append(int(target_argmax[0 if best < 0 else best + 1]))
    return out


def prob_of(dist, x: int) -> float:
    """Total probability of token x under a sparse distribution (ids, probs)."""
    ids, probs = dist
    s = 0.0
    for t, p in zip(ids, probs):
        if int(t) == x:
            s += float(p)
    return s


def residual_weights(p, q) -> list[float]:
    """(p - q)+ over p's support, in p's order (fp64)."""
    ids, probs = p
    return [max(0.0, float(pj) - prob_of(q, int(t))) for t, pj in zip(ids, probs)]


def accept_sampled(p_rows, q_rows, drafts, u) -> list[int]:
    """One sampled window.

    p_rows: k+1 distributions (ids, fp32 probs) for verify rows 0..k;
    q_rows: k draft distributions; drafts: k token ids; u: [k+1][2] fp32.
    """
    out = []
    k = len(drafts)
    for i in range(k):
        x = int(drafts[i])
        px = prob_of(p_rows[i], x)
        qx = prob_of(q_rows[i], x)
        if float(np.float32(u[i][0])) * qx < px:
            out.append(x)
            continue
        r = residual_weights(p_rows[i], q_rows[i])
        z = 0.0
        for w in r:
            z += w
        ids = p_rows[i][0]
        if len(ids) == 0:
            out.append(-1)
        elif z > 0.0:
            out.append(int(ids[draw_weights(r, u[i][1])]))
        else:
            out.append(int(ids[draw(p_rows[i][1], u[i][1])]))
        return out
    ids, probs = p_rows[k]
    out.append(int(ids[draw(probs, u[k][1])]) if len(ids) else -1)
    return out


def accept_point_mass(p_rows, drafts, u) -> list[int]:
    """One window of deterministic drafts under the point-mass rule.

    Row i accepts d_i when u[i][0] < p_i(d_i); otherwise it emits a draw
    (with u[i][1]) from p_i without d_i, renormalised, and ends the window.
    After k acceptances the bonus is drawn from p_k with u[k][1].
    """
    out = []
    k = len(drafts)
    for i in range(k):
        x = int(drafts[i])
        ids, probs = p_rows[i]
        if float(np.float32(u[i][0])) < prob_of(p_rows[i], x):
            out.append(x)
            continue
        w = [0.0 if int(t) == x else float(pj) for t, pj in zip(ids, probs)]
        z = 0.0
        for wj in w:
            z += wj
        if len(ids) == 0:
            out.append(-1)
        elif z > 0.0:
            out.append(int(ids[draw_weights(w, u[i][1])]))
        else:
            out.append(int(ids[draw(probs, u[i][1])]))
        return out
    ids, probs = p_rows[k]
    out.append(int(ids[draw(probs, u[k][1])]) if len(ids) else -1)
    return out


def accept_naive(p_rows, drafts, u) -> list[int]:
    """One window under the naive-sampling verify.

    Row i draws x_i from p_i with u[i][1] and emits it; the window goes on
    while x_i equals d_i, and after k matches emits the bonus draw x_k from
    p_k with u[k][1].  Every emitted token is a draw from its row's p.
    """
    out = []
    k = len(drafts)
    for i in range(k + 1):
        ids, probs = p_rows[i]
        x = int(ids[draw(probs, u[i][1])]) if len(ids) else -1
        out.append(x)
        if i == k or x < 0 or x != int(drafts[i]):
            return out
    return out


def accept_naive_tree(p_rows, tokens, parent, u) -> list[int]:
    """One token tree under the naive-sampling verify (see the module doc).

    p_rows: n + 1 distributions (row 0 = root, row 1 + j = node j); tokens,
    parent: [n] (parent -1 = root); u: [n + 1][2], row r draws with u[r][1].
    """
    n = len(tokens)
    out = []
    node, row = -1, 0
    while True:
        ids, probs = p_rows[row]
        x = int(ids[draw(probs, u[row][1])]) if len(ids) else -1
        out.append(x)
        if x < 0:
            return out
        child = next((j for j in range(n)
                      if -1 <= int(parent[j]) < j and int(parent[j]) == node and int(tokens[j]) == x),
                     None)
        if child is None:
            return out
        node, row = child, child + 1
