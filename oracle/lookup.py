"""Prompt-lookup drafting of a token tree.

[TREE] "One RDNA4 verify pass has slack for about two dozen speculative
tokens": prompt lookup takes the last few emitted tokens, finds where the
same n-gram appeared earlier in the context and proposes what followed it
(the introduction); the tree keeps the top few matches, ranked by how often
they recur, as branches sharing a prefix ("Spend the budget on a tree",
"Where the tree earns its keep", "What I am building toward"), within the
two-dozen-token budget of one verify pass.

Readings taken:
  * the query is the last n tokens of the context; a match is an earlier
    position p (p + n < len, so the query itself is excluded) with
    ctx[p : p + n] equal to the query;
  * a match proposes its continuation ctx[p + n : p + n + depth] (shorter
    where the context ends);
  * identical proposals are one candidate branch whose recurrence count is
    the number of matches proposing it; branches rank by count, then by the
    most recent match (the plain prompt-lookup choice) first;
  * the top `branches` proposals are merged into a trie: walking each in
    rank order from the root, a token already present under the current
    node is shared, otherwise a node is appended (node j's parent is < j;
    -1 is the root, the current position).  Nodes stop at `max_nodes`.
Test infrastructure only.
"""

from __future__ import annotations


def matches(ctx, n: int) -> list[int]:
    """Positions p < len(ctx) - n with ctx[p:p+n] == the last n tokens, most recent first."""
    L = len(ctx)
    if n < 1 or L < n + 1:
        return []
    q = list(ctx[L - n:])
    return [p for p in range(L - n - 1, -1, -1) if list(ctx[p:p + n]) == q]


def ranked_proposals(ctx, n: int, depth: int) -> list[tuple[tuple[int, ...], int, int]]:
    """(continuation, count, most recent position), best first."""
    seen = {}
    for p in matches(ctx, n):  # most recent first
        cont = tuple(int(t) for t in ctx[p + n:p + n + depth])
        if cont in seen:
            seen[cont][0] += 1
        else:
            seen[cont] = [1, p]
    return sorted(((c, cnt, p) for c, (cnt, p) in seen.items()), key=lambda e: (-e[1], -e[2]))


def lookup_tree(ctx, n: int, branches: int, depth: int, max_nodes: int):
    """(tokens, parent) of the drafted tree; empty when nothing matches."""
    tokens, parent = [], []
    for cont, _, _ in ranked_proposals(ctx, n, depth)[:branches]:
        node = -1
        for t in cont:
            child = next((j for j in range(len(tokens)) if parent[j] == node and tokens[j] == t), None)
            if child is None:
                if len(tokens) == max_nodes:
                    return tokens, parent
                tokens.append(t)
                parent.append(node)
                child = len(tokens) - 1
            node = child
    return tokens, parent
