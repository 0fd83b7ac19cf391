"""The acceptance stage of one verify window, stage by stage.

[SD] "Speculative decoding on RDNA": §04 (every verify row, and the draft
step proposed for it, penalised against H_i), §03 (p and q from the same
policy; rejection sampling), §02 (greedy longest-prefix acceptance).

Order: penalise target rows (dense, over the vocabulary) -> top-64 pool ->
policy -> (sampled) penalise and re-score the draft candidates with the
same H_i -> accept.  Also the drafter's own sequential draw of the chain
(each draft drawn from q_i penalised by the drafts before it), used to make
inputs whose drafts really follow q.
"""

from __future__ import annotations

import numpy as np

from .accept import accept_greedy_chain, accept_sampled
from .penalty import penalize_dense, penalize_sparse
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
