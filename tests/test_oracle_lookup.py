"""Pins for the prompt-lookup tree drafter (oracle/lookup.py).

* a hand-worked context whose last n-gram recurs with two different
  continuations, one of them twice: branch order, shared prefix and parents
  written out by hand;
* one branch of ranked matches with no repeated proposal is plain prompt
  lookup: the continuation of the most recent earlier match (brute force);
* every root path of the tree is a prefix of one of the kept proposals, the
  node count is the number of distinct non-empty prefixes, parents precede
  children, and the budget is respected.
"""

import numpy as np

from oracle.lookup import lookup_tree, matches, ranked_proposals


def test_hand_worked_tree():
    ctx = [7, 1, 2, 3, 4, 9, 1, 2, 3, 5, 8, 1, 2, 3, 4, 6, 1, 2]
    # query (n = 2): [1, 2]; earlier matches at 11, 6, 1 (most recent first)
    assert matches(ctx, 2) == [11, 6, 1]
    # proposals (depth 3): 11 -> (3, 4, 6); 6 -> (3, 5, 8); 1 -> (3, 4, 9)
    props = ranked_proposals(ctx, 2, 3)
    assert [p[0] for p in props] == [(3, 4, 6), (3, 5, 8), (3, 4, 9)]
    # depth 2: (3, 4) recurs twice (positions 11 and 1) and outranks (3, 5)
    assert [(p[0], p[1]) for p in ranked_proposals(ctx, 2, 2)] == [((3, 4), 2), ((3, 5), 1)]
    tokens, parent = lookup_tree(ctx, 2, 3, 3, 24)
    # trie: 3 -> 4 -> 6 ; 3 -> 5 -> 8 ; 4 -> 9
    assert tokens == [3, 4, 6, 5, 8, 9]
    assert parent == [-1, 0, 1, 0, 3, 1]
    # budget of 4 nodes: the second branch is cut after its first new node
    assert lookup_tree(ctx, 2, 3, 3, 4) == ([3, 4, 6, 5], [-1, 0, 1, 0])


def most_recent_match_continuation(ctx, n, depth):
    """Plain prompt lookup, written out: scan back for the last n tokens."""
    L = len(ctx)
    for p in range(L - n - 1, -1, -1):
        if all(ctx[p + i] == ctx[L - n + i] for i in range(n)):
            return list(ctx[p + n:p + n + depth])
    return []


def test_single_branch_without_repeats_is_plain_prompt_lookup():
    g = np.random.default_rng(1950)
    for _ in range(300):
        ctx = list(g.integers(0, 6, size=int(g.integers(2, 60))))
        n, depth = int(g.integers(1, 4)), int(g.integers(1, 9))
        props = ranked_proposals(ctx, n, depth)
        if props and props[0][1] == 1:
            tokens, parent = lookup_tree(ctx, n, 1, depth, 64)
            assert tokens == most_recent_match_continuation(ctx, n, depth)
            assert parent == list(range(-1, len(tokens) - 1))


def test_tree_invariants_random():
    g = np.random.default_rng(1951)
    for _ in range(400):
        ctx = list(g.integers(0, 5, size=int(g.integers(2, 200))))
        n, B, D = int(g.integers(1, 4)), int(g.integers(1, 5)), int(g.integers(1, 9))
        budget = int(g.integers(1, 25))
        tokens, parent = lookup_tree(ctx, n, B, D, budget)
        assert len(tokens) <= budget
        assert all(-1 <= parent[j] < j for j in range(len(tokens)))
        kept = [p[0] for p in ranked_proposals(ctx, n, D)[:B]]
        paths = []
        for j in range(len(tokens)):
            path, k = [], j
            while k >= 0:
                path.append(tokens[k])
                k = parent[k]
            paths.append(tuple(reversed(path)))
        assert len(set(paths)) == len(paths)                     # no duplicate siblings
        assert all(any(c[:len(pth)] == pth for c in kept) for pth in paths)
        prefixes = {c[:i] for c in kept for i in range(1, len(c) + 1)}
        if budget >= 64 or len(prefixes) <= budget:
            assert set(paths) == prefixes
