"""Windowed repeat / frequency / presence penalties on every verify row.

[SD] "Speculative decoding on RDNA", §04 "Penalties on every verify row",
figure "the penalty history of verify row i": verify row i is penalised
against H_i, the last W tokens of (prompt || emitted so far || drafts
[0, i)); a draft enters the history of the rows after it, and both the
target row p_i and the draft step q_i use the same H_i.

The pages name the three penalties but print no formulas.  The reading
taken here (one window W for all three):
  for each distinct token t in H_i with count c >= 1, on logit l of t:
    l1 = l / repeat   if l > 0   else  l * repeat
    l2 = l1 - c * frequency
    l3 = l2 - presence
evaluated in fp32, one rounding per operation, in that order, with no
fused multiply-add (the page calls the GPU prepass bit-identical to the
host stage, which fixes an exact op sequence).  W = 0 means no penalties;
a shorter history uses every token available; ids outside [0, V) are
ignored.

Token trees ([TREE] "Spend the budget on a tree": each branch attends only
to its own ancestors): the same rule applied per branch.  Row 0 is the
root (the current position) with H = last W of the context; row 1 + j is
node j with H = last W of (context || the tokens on the path from the root
down to node j, inclusive).  A chain (parent[j] = j - 1) gives the chain's
H_{j+1}.  A parent outside [-1, j) ends the path as the root would.
"""

from __future__ import annotations

from collections import Counter

import numpy as np


def history(ctx: np.ndarray, drafts: np.ndarray, i: int, window: int) -> list[int]:
    """H_i = last `window` tokens of (ctx || drafts[0, min(i, len(drafts))))."""
    if window <= 0:
        return []
    seq = [int(t) for t in ctx] + [int(t) for t in drafts[:min(i, len(drafts))]]
    return seq[-window:] if len(seq) > window else seq


def tree_path(tokens, parent, j: int) -> list[int]:
    """Tokens from the root's child down to node j (inclusive)."""
    path = [int(tokens[j])]
    child, q = j, int(parent[j])
    while -1 < q < child:
        path.append(int(tokens[q]))
        child, q = q, int(parent[q])
    path.reverse()
    return path


def tree_history(ctx, tokens, parent, row: int, window: int) -> list[int]:
    """Row 0: last `window` of ctx; row 1 + j: last `window` of ctx || tree_path(j)."""
    if window <= 0:
        return []
    seq = [int(t) for t in ctx] + (tree_path(tokens, parent, row - 1) if row > 0 else [])
    return seq[-window:] if len(seq) > window else seq


def penalize_value(l: np.float32, c: int, repeat: np.float32, presence: np.float32,
                   frequency: np.float32) -> np.float32:
    """One penalised logit, fp32 ops in the order stated in the module doc."""
    l = np.float32(l)
    rep, pres, freq = np.float32(repeat), np.float32(presence), np.float32(frequency)
    with np.errstate(all="ignore"):
        l1 = np.float32(l / rep) if l > np.float32(0) else np.float32(l * rep)
        cf = np.float32(np.float32(c) * freq)
        l2 = np.float32(l1 - cf)
        l3 = np.float32(l2 - pres)
    return l3


def penalize_dense(logits: np.ndarray, ctx: np.ndarray, drafts: np.ndarray, window: int,
                   repeat: float, presence: float, frequency: float) -> np.ndarray:
    """Row i of logits [rows][V] (fp32) is penalised by H_i.  Returns a copy."""
    out = np.array(logits, dtype=np.float32, copy=True)
    V = out.shape[1]
    for i in range(out.shape[0]):
        counts = Counter(history(ctx, drafts, i, window))
        for t, c in counts.items():
            if 0 <= t < V:
                out[i, t] = penalize_value(out[i, t], c, repeat, presence, frequency)
    return out


def penalize_sparse(ids: np.ndarray, vals: np.ndarray, ctx: np.ndarray, drafts: np.ndarray,
                    window: int, repeat: float, presence: float, frequency: float, *,
                    vocab: int) -> np.ndarray:
    """Candidate lists: row i holds ids[i][m] with logits vals[i][m].

    Each candidate slot whose id occurs in H_i is penalised with that id's
    count; tokens of H_i outside [0, vocab) are ignored, as for dense rows,
    so a slot holding such an id (an empty slot, for instance) is never
    penalised.  Used for the draft's re-scored candidates, which get the
    same H_i as the target row.  Returns a copy of vals.
    """
    out = np.array(vals, dtype=np.float32, copy=True)
    for i in range(out.shape[0]):
        counts = Counter(t for t in history(ctx, drafts, i, window) if 0 <= t < vocab)
        for m in range(out.shape[1]):
            c = counts.get(int(ids[i, m]), 0)
            if c >= 1:
                out[i, m] = penalize_value(out[i, m], c, repeat, presence, frequency)
    return out


def penalize_tree_dense(logits, ctx, tokens, parent, window: int, repeat: float, presence: float,
                        frequency: float) -> np.ndarray:
    """Rows [n_nodes + 1][V]: row r penalised by tree_history(r).  Returns a copy."""
    out = np.array(logits, dtype=np.float32, copy=True)
    V = out.shape[1]
    for r in range(out.shape[0]):
        counts = Counter(tree_history(ctx, tokens, parent, r, window))
        for t, c in counts.items():
            if 0 <= t < V:
                out[r, t] = penalize_value(out[r, t], c, repeat, presence, frequency)
    return out


def penalize_tree_sparse(ids, vals, ctx, tokens, parent, window: int, repeat: float,
                         presence: float, frequency: float, *, vocab: int) -> np.ndarray:
    """Candidate lists per tree row, penalised with tree_history(r) (its
    tokens outside [0, vocab) ignored).  Returns a copy of vals."""
    out = np.array(vals, dtype=np.float32, copy=True)
    for r in range(out.shape[0]):
        counts = Counter(t for t in tree_history(ctx, tokens, parent, r, window) if 0 <= t < vocab)
        for m in range(out.shape[1]):
            c = counts.get(int(ids[r, m]), 0)
            if c >= 1:
                out[r, m] = penalize_value(out[r, m], c, repeat, presence, frequency)
    return out
