"""GPU parity of tree_attention_rows and tree_commit_kv against the oracle.

[TREE] "Spend the budget on a tree, not a longer guess" (the tree attention
mask: each branch attends only to its ancestors) and "Where the tree earns
its keep" (candidate keys and values in scratch slots; only the accepted
branch is kept).

Tolerance: every output element within 1e-4 * sum_j softmax_j * |v_j| of the
fp64 oracle.  The kernel's products are exact (queries and probabilities
split into three bf16 pieces); its fp32 sums run over 128 head dimensions,
one 64-key block and the blocks of a split ((128 + 64 + 64) * 2^-24 ~
1.5e-5 relative), and its exponential is the hardware base-2 one after one
rounded multiply by log2(e) (relative error about |x| * 2^-24 + 2^-23 for
an exponent |x| below ~40 here, ~3e-6): together a few 1e-5 of that
magnitude at most.  The observed worst is ~1.4e-7.  The commit is bit-exact.
"""

import numpy as np
import pytest
import torch

import verify_sampling_amd as vs
from gpu_common import dev, host
from oracle.tree_attention import commit_branch, tree_attention
from synth import f32_to_bf16_bits

pytestmark = pytest.mark.gpu


def case(seed, R, Hq, Hkv, ctx, L=None, D=128):
    g = np.random.default_rng(seed)
    L = L if L is not None else ctx + R + 8
    q = g.standard_normal((R, Hq, D)).astype(np.float32)
    kc = f32_to_bf16_bits(g.standard_normal((Hkv, L, D)).astype(np.float32))
    vc = f32_to_bf16_bits(g.standard_normal((Hkv, L, D)).astype(np.float32))
    ks = f32_to_bf16_bits(g.standard_normal((Hkv, R, D)).astype(np.float32))
    vs_ = f32_to_bf16_bits(g.standard_normal((Hkv, R, D)).astype(np.float32))
    return q, kc, vc, ks, vs_


def tree_3x8():
    """3 branches x depth 8: 24 nodes, node 8 b + d at depth d + 1 of branch b."""
    parent = []
    for b in range(3):
        for d in range(8):
            parent.append(-1 if d == 0 else len(parent) - 1)
    return np.array(parent, dtype=np.int32)


def run(q, kc, vc, ctx, ks, vs_, parent, scale):
    out = vs.tree_attention_rows(dev(q), dev(kc), dev(vc), ctx, dev(ks), dev(vs_),
                                 dev(parent) if len(parent) else None, scale=scale)
    return host(out)


def check(got, q, kc, vc, ctx, ks, vs_, parent, scale):
    want, s_abs = tree_attention(q, kc, vc, ctx, ks, vs_, parent, scale)
    err = np.abs(got.astype(np.float64) - want)
    ratio = float((err / (s_abs + 1e-30)).max())
    assert (err <= 1e-4 * s_abs).all(), ratio
    return ratio


def test_three_branch_depth_eight_tree_over_a_long_context():
    """The 24-node tree (3 branches x depth 8) of an 8B-class layer: 32 query
    heads, 8 KV heads, head dimension 128, 2080 context positions."""
    R, Hq, Hkv, ctx = 25, 32, 8, 2080
    q, kc, vc, ks, vs_ = case(2200, R, Hq, Hkv, ctx)
    parent = tree_3x8()
    got = run(q, kc, vc, ctx, ks, vs_, parent, 1 / np.sqrt(128))
    print("worst error / (sum p |v|):", check(got, q, kc, vc, ctx, ks, vs_, parent, 1 / np.sqrt(128)))


@pytest.mark.parametrize("ctx", [0, 1, 63, 64, 65, 200, 1000])
def test_ragged_contexts_and_random_trees(ctx):
    g = np.random.default_rng(2210 + ctx)
    n = 12
    parent = np.array([-1] + [int(g.integers(-1, j)) for j in range(1, n)], dtype=np.int32)
    R, Hq, Hkv = n + 1, 8, 2
    q, kc, vc, ks, vs_ = case(2220 + ctx, R, Hq, Hkv, ctx)
    got = run(q, kc, vc, ctx, ks, vs_, parent, 0.09)
    check(got, q, kc, vc, ctx, ks, vs_, parent, 0.09)


def test_chain_root_only_and_malformed_parents():
    R, Hq, Hkv, ctx = 9, 4, 4, 70
    q, kc, vc, ks, vs_ = case(2230, R, Hq, Hkv, ctx)
    chain = np.arange(-1, R - 2, dtype=np.int32)
    check(run(q, kc, vc, ctx, ks, vs_, chain, 0.1), q, kc, vc, ctx, ks, vs_, chain, 0.1)
    bad = np.array([-1, 5, 0, -9, 2, 2, 7, 100], dtype=np.int32)  # parents outside [-1, j) cut the path
    check(run(q, kc, vc, ctx, ks, vs_, bad, 0.1), q, kc, vc, ctx, ks, vs_, bad, 0.1)
    q1, kc1, vc1, ks1, vs1 = case(2231, 1, 4, 2, 33)  # the root alone
    check(run(q1, kc1, vc1, 33, ks1, vs1, np.zeros(0, np.int32), 0.1), q1, kc1, vc1, 33, ks1, vs1, [], 0.1)


def test_most_rows_and_repeatability():
    """64 rows with 4 query heads per KV head (256 queries per KV head, the
    most a call takes); two calls give the same bits."""
    g = np.random.default_rng(2240)
    n = 63
    parent = np.array([-1] + [int(g.integers(max(-1, j - 4), j)) for j in range(1, n)], dtype=np.int32)
    R, Hq, Hkv, ctx = n + 1, 8, 2, 300
    q, kc, vc, ks, vs_ = case(2241, R, Hq, Hkv, ctx)
    a = run(q, kc, vc, ctx, ks, vs_, parent, 0.08)
    b = run(q, kc, vc, ctx, ks, vs_, parent, 0.08)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    check(a, q, kc, vc, ctx, ks, vs_, parent, 0.08)


def test_commit_keeps_the_accepted_branch():
    R, Hq, Hkv, ctx, L = 25, 8, 8, 500, 600
    _, kc, vc, ks, vs_ = case(2250, R, Hq, Hkv, ctx, L)
    path = np.array([0, 9, 10, 11, 12], dtype=np.int32)  # root, then branch 1 to depth 4
    K, V = dev(kc), dev(vc)
    vs.tree_commit_kv(K, V, ctx, dev(ks), dev(vs_), dev(path))
    want_k, want_v = commit_branch(kc, vc, ctx, ks, vs_, path)
    assert np.array_equal(host(K), want_k) and np.array_equal(host(V), want_v)
    # an invalid slot index leaves its position unchanged
    K2, V2 = dev(kc), dev(vc)
    vs.tree_commit_kv(K2, V2, ctx, dev(ks), dev(vs_), dev(np.array([0, 99, 3], dtype=np.int32)))
    k2 = host(K2)
    assert np.array_equal(k2[:, ctx], ks[:, 0]) and np.array_equal(k2[:, ctx + 1], kc[:, ctx + 1])
    assert np.array_equal(k2[:, ctx + 2], ks[:, 3])


@pytest.mark.parametrize("seed", range(2300, 2312))
def test_random_trees_heads_and_contexts(seed):
    """Seeded random shapes: rows 1..64, query heads per KV head 1..8 (at most
    256 queries per KV head), 1..8 KV heads, contexts 0..3000 (ragged last
    blocks), random parents (some malformed), scales, and scratch longer than
    the tree; every output within the tolerance of the oracle."""
    g = np.random.default_rng(seed)
    Hkv = int(g.choice([1, 2, 4, 8]))
    G = int(g.choice([1, 2, 4, 8]))
    R = int(g.integers(1, min(64, 256 // G) + 1))
    ctx = int(g.choice([0, 1, 31, 64, 129, 777, 2080, 3000]))
    parent = np.array([int(g.integers(-1, j)) if j > 0 else -1 for j in range(R - 1)], dtype=np.int32)
    if R > 3 and g.integers(0, 3) == 0:
        parent[int(g.integers(1, R - 1))] = int(g.choice([-7, R + 3]))   # a malformed parent
    scale = float(g.uniform(0.02, 0.2))
    print(f"seed {seed}: R={R} G={G} Hkv={Hkv} ctx={ctx}", flush=True)
    q, kc, vc, ks, vs_ = case(seed + 100, R, G * Hkv, Hkv, ctx, L=ctx + 1 + int(g.integers(0, 40)))
    ks_long = np.concatenate([ks, ks[:, :2]], axis=1)   # scratch of R + 2 slots
    vs_long = np.concatenate([vs_, vs_[:, :2]], axis=1)
    got = run(q, kc, vc, ctx, ks_long, vs_long, parent, scale)
    check(got, q, kc, vc, ctx, ks_long, vs_long, parent, scale)


@pytest.mark.parametrize("R,G,Hkv,ctx", [(9, 4, 8, 8000), (5, 4, 1, 40000), (9, 2, 16, 2000)])
def test_long_contexts_walk_several_sub_blocks_per_split(R, G, Hkv, ctx):
    """Long contexts: each split walks three or four 64-key sub-blocks (8000
    positions over 8 KV heads, 40000 over one), the next in flight while the
    current one is computed, and many splits are merged (210 for 40000)."""
    g = np.random.default_rng(2400 + ctx)
    parent = np.array([int(g.integers(-1, j)) if j > 0 else -1 for j in range(R - 1)], dtype=np.int32)
    q, kc, vc, ks, vs_ = case(2410 + Hkv, R, G * Hkv, Hkv, ctx)
    check(run(q, kc, vc, ctx, ks, vs_, parent, 0.07), q, kc, vc, ctx, ks, vs_, parent, 0.07)
