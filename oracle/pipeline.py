"""The acceptance stage of one verify window, stage by stage (a chain of
drafts, or a token tree).

[SD] "Speculative decoding on RDNA": §04 (every verify row, and the draft
step proposed for it, penalised against H_i), §03 (p and q from the same
policy; rejection sampling), §02 (greedy longest-prefix acceptance).

Order: penalise target rows (dense, over the vocabulary) -> top-64 pool ->
policy -> (sampled) penalise and re-score the draft candidates with the
same H_i -> accept.  Also the drafter's own sequential draw of the chain
(each draft drawn from q_i penalised by the drafts before it), used to make
inputs whose drafts really follow q.

A token tree ([TREE] "Spend the budget on a tree, not a longer guess":
one pass verifies several branches sharing a prefix) takes the same
stages with one history per row: row 0 (the root) the context, row 1 + j
(node j) the context followed by the path from the root down to node j,
so each branch is penalised as its own chain would be; then the pool and
the policy per row, then the greedy tree walk or the naive-sampling walk
(deterministic drafts: draw from the row's p, follow the child holding the
drawn token).
"""

from __future__ import annotations

import numpy as np

from .accept import accept_greedy_chain, accept_greedy_tree, accept_naive_tree, accept_sampled
from .penalty import penalize_dense, penalize_sparse, penalize_tree_dense
from .policy import POOL, draw, policy_row
from .topk import topk_rows


def draft_chain(q_ids, q_vals, ctx, u_draft, *, vocab, window, repeat, presence, frequency,
                temperature, top_k, top_p, min_p):
    """Draw d_0..d_{k-1}; d_i ~ q_i, with q_i penalised by H_i (which holds d_0..d_{i-1})."""
    k = q_ids.shape[0]
    drafts = np.zeros(k, dtype=np.int32)
    for i in range(k):
        # row i of the candidates is penalised by H_i = ctx || drafts[:i]
        pen = penalize_sparse(q_ids, q_vals, ctx, drafts[:i], window, repeat, presence, frequency,
                              vocab=vocab)[i]
        ids, probs = policy_row(pen, q_ids[i], temperature, top_k, top_p, min_p)
        drafts[i] = ids[draw(probs, u_draft[i])]
    return drafts


def acceptance_stage(target_logits, ctx, drafts, u, *, q_ids=None, q_vals=None, window, repeat,
                     presence, frequency, temperature, top_k, top_p, min_p, pool=POOL):
    """One window: target_logits fp32 [k+1][V]; drafts [k]; u fp32 [k+1][2].

    Greedy when temperature <= 0 (q not needed).  Returns a dict with the
    penalised rows, the pools, the distributions and the emitted tokens.
    """
    k = len(drafts)
    pen = penalize_dense(target_logits, ctx, drafts, window, repeat, presence, frequency)
    pool_vals, pool_ids = topk_rows(pen, pool)
    p_rows = [policy_row(pool_vals[i], pool_ids[i], temperature, top_k, top_p, min_p)
              for i in range(k + 1)]
    out = {"penalized": pen, "pool_vals": pool_vals, "pool_ids": pool_ids, "p_rows": p_rows}
    if float(np.float32(temperature)) <= 0.0:
        out["tokens"] = accept_greedy_chain(pool_ids[:, 0], drafts)
        return out
    q_pen = penalize_sparse(q_ids, q_vals, ctx, drafts, window, repeat, presence, frequency,
                            vocab=target_logits.shape[1])
    q_rows = [policy_row(q_pen[i], q_ids[i], temperature, top_k, top_p, min_p) for i in range(k)]
    out["q_penalized"] = q_pen
    out["q_rows"] = q_rows
    out["tokens"] = accept_sampled(p_rows, q_rows, drafts, u)
    return out


def tree_acceptance_stage(target_logits, ctx, tokens, parent, u, *, window, repeat, presence,
                          frequency, temperature, top_k, top_p, min_p, pool=POOL):
    """One token tree: target_logits fp32 [n+1][V] (row 0 the root, row 1 + j
    node j); tokens, parent [n] (parent -1 = the root); u fp32 [n+1][2].

    Each row penalised with its own branch's history, then the pool, the
    policy, and the greedy tree walk (temperature <= 0) or the
    naive-sampling walk.  Returns the penalised rows, pools, distributions
    and emitted tokens.
    """
    n = len(tokens)
    pen = penalize_tree_dense(target_logits, ctx, tokens, parent, window, repeat, presence, frequency)
    pool_vals, pool_ids = topk_rows(pen, pool)
    p_rows = [policy_row(pool_vals[r], pool_ids[r], temperature, top_k, top_p, min_p)
              for r in range(n + 1)]
    out = {"penalized": pen, "pool_vals": pool_vals, "pool_ids": pool_ids, "p_rows": p_rows}
    if float(np.float32(temperature)) <= 0.0:
        out["tokens"] = accept_greedy_tree(pool_ids[:, 0], tokens, parent)
    else:
        out["tokens"] = accept_naive_tree(p_rows, tokens, parent, u)
    return out
