"""verify_tree_window (a token tree's acceptance stage in two launches)
against the separate calls it replaces, byte for byte, and against the
oracle's composition on seeded logits.

[TREE] "Spend the budget on a tree, not a longer guess": several branches
sharing a prefix, each seeing only its ancestors; "Speculative decoding on
RDNA" §04 (each row penalised against its own history), §03 (pool and
policy); [PR] "Code map" (the naive-sampling verify, walked down the tree).
The separate sequence is penalize_tree_rows, topk_rows at K = 64,
sample_policy_rows and spec_accept_rows (naive-sampling or greedy tree
walk); every output of the fused call (penalised logits, pools,
distributions, tokens) must carry the same bits.  Cases cover a 3 x 8 tree
on LM-head rows, random trees with malformed parents and ids outside the
vocabulary, a 63-node chain, the root alone, both chunk sizes of the pool
selection and a single chunk, long and empty windows, unaligned rows and
planted hard logits.
"""

import numpy as np
import pytest
import torch

import verify_sampling_amd as vs
from gpu_common import host
from oracle.pipeline import tree_acceptance_stage
from synth import logits, penalty_history, topk_planted_rows, tree_window, uniforms

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CFG = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)
PEN = dict(window=64, repeat=1.1, presence=1.5, frequency=0.2)


def make_tree(seed, V, R, *, kind="random", ctx_len=2080, ld=None, planted=False, bad=False):
    """Seeded tree inputs: logits [R][ld] (V valid), history, tokens and
    parents of the R - 1 nodes, uniforms [R][2]."""
    n = R - 1
    ld = ld or V
    g = np.random.default_rng(seed)
    if kind == "3x8":
        x, ctx, tokens, parent, u = tree_window(seed, V)
        ctx = ctx[:ctx_len]
    else:
        x = topk_planted_rows(seed, rows=R, vocab=V, K=64) if planted else logits(seed, (R, V))
        if kind == "chain":
            parent = np.arange(-1, n - 1, dtype=np.int32)
        else:
            parent = np.array([int(g.integers(-1, j)) if j > 0 else -1 for j in range(n)], dtype=np.int32)
        tokens = np.zeros(n, dtype=np.int32)
        for j in range(n):  # mostly one of the parent row's top few, so that walks go on
            prow = 0 if parent[j] < 0 else parent[j] + 1
            top = np.argsort(-np.nan_to_num(x[prow], nan=-np.inf), kind="stable")[:4]
            tokens[j] = int(top[g.integers(0, 4)]) if g.random() < 0.8 else int(g.integers(0, V))
        if bad and n > 4:
            parent[n // 2] = n + 3            # malformed: ends that node's path
            parent[n - 1] = -7
            tokens[1] = V + 2                 # outside the vocabulary: never penalised, never drawn
        hot = np.unique(np.argsort(-np.nan_to_num(x, nan=-np.inf), axis=1)[:, :64])
        ctx = penalty_history(seed + 1, V, max(ctx_len - 32, 0), min(ctx_len, 32), hot)[:ctx_len]
        if bad and ctx_len >= 8:
            ctx[[1, 5, ctx_len - 2]] = [-3, V + 5, V]
        u = uniforms(seed + 4, (R, 2))
    lg = np.zeros((R, ld), dtype=np.float32)
    lg[:, :V] = x
    return lg, ctx, tokens, parent, u


def to_dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


def separate(lg, ctx, tokens, parent, u, V, pen, cfg):
    L, C, T, P, U = to_dev(lg, ctx, tokens, parent, u)
    Lv = L[:, :V]
    vs.penalize_tree_rows(Lv, C, T, P, **pen)
    pv, pi = vs.topk_rows(Lv, 64)
    p = vs.sample_policy_rows(pv, pi, **cfg)[:3]
    sampled = cfg["temperature"] > 0
    mode = vs.ACCEPT_NAIVE_TREE if sampled else vs.ACCEPT_GREEDY_TREE
    tok, n = vs.spec_accept_rows(mode, T[None, :], p, u=U[None] if sampled else None, parent=P[None, :])
    return dict(logits=L, pool_vals=pv, pool_ids=pi, p=p, tokens=tok[0], n=n)


def fused(lg, ctx, tokens, parent, u, V, pen, cfg, workspace=None):
    L, C, T, P, U = to_dev(lg, ctx, tokens, parent, u)
    out = vs.verify_tree_window(L[:, :V], C, T, P, u=U, workspace=workspace, **pen, **cfg)
    out["logits"] = L
    return out


def bits(t):
    a = host(t)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_same(a, b):
    assert np.array_equal(bits(a["logits"]), bits(b["logits"])), "penalised logits"
    assert np.array_equal(bits(a["pool_vals"]), bits(b["pool_vals"])), "pool values"
    assert np.array_equal(bits(a["pool_ids"]), bits(b["pool_ids"])), "pool ids"
    for x, y, name in zip(a["p"], b["p"], ("p_ids", "p_probs", "p_len")):
        assert np.array_equal(bits(x), bits(y)), name
    n = int(host(a["n"])[0])
    assert n == int(host(b["n"])[0])
    tk_a, tk_b = host(a["tokens"]), host(b["tokens"])
    assert np.array_equal(tk_a[:n], tk_b[:n]), "tokens"
    assert (tk_a[n:] == -1).all()
    assert 1 <= n <= len(tk_a)


CASES = {
    # name: (seed, V, R, make_tree options, penalty options, policy options)
    "lm_head_3x8": (3300, 151936, 25, dict(kind="3x8"), {}, {}),
    "lm_head_3x8_greedy": (3310, 151936, 25, dict(kind="3x8"), {}, dict(temperature=0.0)),
    "lm_head_3x8_t1": (3320, 151936, 25, dict(kind="3x8"), {}, dict(temperature=1.0, top_k=0, top_p=1.0,
                                                                     min_p=0.0)),
    "window_0": (3330, 151936, 9, {}, dict(window=0), {}),
    "long_window_hash_counts": (3340, 151936, 9, dict(ctx_len=6000), dict(window=4096), {}),
    "no_context": (3350, 151936, 5, dict(ctx_len=0), {}, {}),
    "root_only": (3360, 151936, 1, {}, {}, {}),
    "root_only_greedy": (3365, 151936, 1, {}, {}, dict(temperature=0.0)),
    "chain_of_63": (3370, 151936, 64, dict(kind="chain"), {}, {}),
    "chain_of_63_window_32": (3375, 151936, 64, dict(kind="chain"), dict(window=32), dict(temperature=0.0)),
    "random_malformed": (3380, 151936, 25, dict(bad=True), {}, {}),
    "random_malformed_greedy": (3385, 151936, 25, dict(bad=True), {}, dict(temperature=0.0)),
    "one_chunk_v1000": (3390, 1000, 9, {}, {}, {}),
    "v4096_r16": (3400, 4096, 16, {}, dict(window=300), dict(temperature=1.3, top_k=64)),
    "unaligned_rows": (3410, 50257, 12, dict(ld=50260), {}, {}),
    "planted_hard_rows": (3420, 151936, 9, dict(planted=True, bad=True), {}, {}),
    "negative_penalties": (3430, 151936, 9, {}, dict(presence=-0.5, frequency=-0.25, repeat=0.8), {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_tree_window_equals_separate_calls(name):
    seed, V, R, opts, pen_o, cfg_o = CASES[name]
    lg, ctx, tokens, parent, u = make_tree(seed, V, R, **opts)
    pen, cfg = dict(PEN, **pen_o), dict(CFG, **cfg_o)
    a = fused(lg, ctx, tokens, parent, u, V, pen, cfg)
    b = separate(lg, ctx, tokens, parent, u, V, pen, cfg)
    assert_same(a, b)
    print(f"{name}: emitted {int(host(a['n'])[0])}")


def test_workspace_reused_across_trees():
    """One workspace, sized for the largest need, serves trees of every size
    in turn (the arrival counter is reset by each call's first launch)."""
    V = 151936
    trees = ((3440, 64), (3441, 9), (3442, 25), (3443, 2), (3444, 64))
    # the pool's chunk size depends on the row count, so the largest need is not the largest tree's
    need = max(vs.verify_window_workspace_bytes(R, V) for _, R in trees)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    for seed, R in trees:
        lg, ctx, tokens, parent, u = make_tree(seed, V, R)
        a = fused(lg, ctx, tokens, parent, u, V, PEN, CFG, workspace=ws)
        b = separate(lg, ctx, tokens, parent, u, V, PEN, CFG)
        assert_same(a, b)


@pytest.mark.parametrize("seed,V,temperature", [(3450, 4096, 0.7), (3460, 4096, 0.0), (3470, 151936, 0.7)])
def test_fused_tree_window_equals_oracle(seed, V, temperature):
    """The oracle's composition on the same fp32 logits: penalised rows and
    pools bit for bit, the same tokens."""
    lg, ctx, tokens, parent, u = make_tree(seed, V, 25, kind="3x8" if V == 151936 else "random")
    cfg = dict(CFG, temperature=temperature)
    got = fused(lg, ctx, tokens, parent, u, V, PEN, cfg)
    want = tree_acceptance_stage(lg[:, :V], ctx, tokens, parent, u, **PEN, **cfg)
    assert np.array_equal(bits(got["logits"])[:, :V], want["penalized"].view(np.uint32))
    assert np.array_equal(bits(got["pool_ids"]), want["pool_ids"])
    assert np.array_equal(bits(got["pool_vals"]), want["pool_vals"].view(np.uint32))
    n = int(host(got["n"])[0])
    assert [int(t) for t in host(got["tokens"])[:n]] == [int(t) for t in want["tokens"]]
