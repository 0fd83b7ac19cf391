"""Attention of a token tree's verify rows, and the commit of the accepted branch.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[TREE] "One RDNA4 verify pass has slack for about two dozen speculative
tokens":
  * "Spend the budget on a tree, not a longer guess": several continuations
    that share a prefix are verified in one pass, with a tree-shaped
    attention mask under which every branch attends only to its own
    ancestors;
  * "Where the tree earns its keep, and where it does not": the candidates'
    keys and values are written to scratch slots and only the accepted
    branch is kept;
  * "What I am building toward": the mask is folded into the decode kernel.

Readings taken (the pages give no formulas):
  * rows and slots: row 0 is the root, the current position, whose key and
    value are in scratch slot 0; row 1 + j is tree node j, in slot 1 + j.
    Node j's parent is parent[j] (-1 = the root); the path from node j up
    stops at the root or at a parent outside [-1, child), as for the tree
    penalty histories, so a malformed parent leaves the node below the root;
  * row r attends to every context position [0, ctx_len) of the KV cache and
    to the scratch slots of its ancestors and itself: {0} for the root,
    {0} + {1 + a : a on node j's path, j included} for row 1 + j.  A chain
    (parent[j] = j - 1) is causal attention over context || slots 0..r;
  * scores s = scale * (q . k), softmax over the allowed keys, output
    sum_j softmax_j * v_j, all in fp64 from fp32 queries and bf16 keys and
    values (decoded exactly: bits << 16);
  * grouped heads: query head h reads KV head h // (Hq / Hkv);
  * commit: the accepted path, as slot indices root first (0, then the
    slots of the accepted nodes in order), is copied into the cache at
    positions ctx_len, ctx_len + 1, ... for every KV head, bits unchanged;
    nothing else in the cache changes.

Layouts: q float32 [R][Hq][D]; k_cache, v_cache uint16 (bf16 bits)
[Hkv][L][D]; k_scr, v_scr uint16 [Hkv][S][D] with S >= R; out [R][Hq][D].
"""

from __future__ import annotations

import numpy as np


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def row_slots(parent, row: int) -> list[int]:
    """Scratch slots row `row` attends to, root first."""
    if row == 0:
        return [0]
    child = row - 1
    path = [child]
    q = int(parent[child])
    while -1 < q < child:
        path.append(q)
        child, q = q, int(parent[q])
    return [0] + [1 + a for a in reversed(path)]


def tree_attention(q, k_cache, v_cache, ctx_len: int, k_scr, v_scr, parent, scale: float):
    """out float64 [R][Hq][D] and s_abs [R][Hq][D] = sum_j softmax_j * |v_j| (the
    magnitude the tolerance is taken against)."""
    q = np.asarray(q, dtype=np.float32).astype(np.float64)
    R, Hq, D = q.shape
    Hkv = k_cache.shape[0]
    group = Hq // Hkv
    kc, vc = bf16_to_f64(k_cache), bf16_to_f64(v_cache)
    ks, vs = bf16_to_f64(k_scr), bf16_to_f64(v_scr)
    out = np.zeros((R, Hq, D))
    s_abs = np.zeros((R, Hq, D))
    for r in range(R):
        slots = row_slots(parent, r)
        for h in range(Hq):
            g = h // group
            keys = np.concatenate([kc[g, :ctx_len], ks[g, slots]], axis=0)
            vals = np.concatenate([vc[g, :ctx_len], vs[g, slots]], axis=0)
            s = scale * (keys @ q[r, h])
            w = np.exp(s - s.max())
            p = w / w.sum()
            out[r, h] = p @ vals
            s_abs[r, h] = p @ np.abs(vals)
    return out, s_abs


def commit_branch(k_cache, v_cache, ctx_len: int, k_scr, v_scr, path_slots):
    """Copies of the caches with the accepted path's slots written at
    positions ctx_len, ctx_len + 1, ... (every KV head)."""
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    for i, s in enumerate(path_slots):
        kc[:, ctx_len + i] = k_scr[:, int(s)]
        vc[:, ctx_len + i] = v_scr[:, int(s)]
    return kc, vc
