"""GPU parity of verify_windows, the batched sampled acceptance stage in one launch.

"Speculative decoding on RDNA", §03: each window's target and draft rows
are pooled (top 64) and turned into the policy distribution (temperature,
top-k, min-p, top-p); the drafts are draws from q; acceptance is rejection
sampling with the residual and bonus draws.

Two ways:
- against the five separate calls (topk_rows and sample_policy_rows on the
  target rows, the same two on the draft rows with the drafts' uniforms,
  spec_accept_rows): every output byte for byte, over seeded configurations
  (batch sizes on both sides of the one-launch limit, draft counts,
  vocabularies of 64 to 4096, padded rows, policy settings, rows with ties,
  NaN and -inf);
- against the oracle stage by stage: the distributions equal the oracle's
  policy on the oracle's pool (ids and lengths exactly, probabilities within
  1 fp32 ulp), the drafts equal the oracle's draws from the GPU's q rows, and
  the tokens equal the oracle's acceptance of the GPU's distributions; and
  the first emitted token of 200,000 windows over one repeated set of rows
  follows p_0 (chi-square).
"""

import numpy as np
import pytest
import torch

import verify_sampling_amd as vs
from gpu_common import dev, host, ulp_diff_f32
from oracle.accept import accept_sampled
from oracle.policy import draw, policy_row
from oracle.topk import topk_rows
from stats import chi2_pvalue
from synth import correlated_logits, logits, rng, uniforms

pytestmark = pytest.mark.gpu
CFG = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)


def special_rows(x, seed):
    """Plants row kinds the pool order must handle into some rows of x."""
    g = rng(seed)
    n, V = x.shape
    for r in g.choice(n, size=min(n, 12), replace=False):
        kind = int(g.integers(0, 6))
        if kind == 0:
            x[r] = np.float32(1.5)                                   # all equal
        elif kind == 1:
            x[r, g.choice(V, V // 2, replace=False)] = -np.inf       # half -inf
        elif kind == 2:
            x[r, g.choice(V, 8, replace=False)] = np.nan             # NaN entries
        elif kind == 3:
            x[r] = np.round(x[r])                                    # integer ties
        elif kind == 4:
            x[r] = -np.inf
            x[r, g.choice(V, 3, replace=False)] = 0.25               # three finite values
        else:
            top = int(np.argmax(x[r]))
            x[r, g.choice(V, 5, replace=False)] = x[r, top]          # repeated maximum
    return x


def case(seed, B, k, V, pad=0, special=True):
    p = logits(seed, (B * (k + 1), V))
    q = correlated_logits(p.reshape(B, k + 1, V)[:, :k].reshape(B * k, V), 0.8, seed + 1) if k else \
        np.zeros((0, V), np.float32)
    if special:
        p = special_rows(p, seed + 2)
        if k:
            q = special_rows(q, seed + 3)
    if pad:
        p = np.pad(p, ((0, 0), (0, pad)), constant_values=np.float32(7.0))  # never read
        q = np.pad(q, ((0, 0), (0, pad)), constant_values=np.float32(7.0))
    u = uniforms(seed + 4, (B, k + 1, 2))
    ud = uniforms(seed + 5, (max(1, B * k),))[:B * k]
    return p, q, u, ud


def separate(P, Q, k, V, U, UD, cfg):
    """The five separate calls verify_windows stands for."""
    B = P.shape[0] // (k + 1)
    Pv = P[:, :V]
    pv, pi = vs.topk_rows(Pv, 64)
    pd = vs.sample_policy_rows(pv, pi, **cfg)[:3]
    if k:
        qv, qi = vs.topk_rows(Q[:, :V], 64)
        qids, qprobs, qlen, drafts = vs.sample_policy_rows(qv, qi, u=UD, **cfg)
        qd = (qids, qprobs, qlen)
    else:
        qd, drafts = None, torch.empty((0,), dtype=torch.int32, device=P.device)
    tok, n = vs.spec_accept_rows(vs.ACCEPT_SAMPLED, drafts.view(B, k), pd, qd, u=U)
    return tok, n, drafts, pd, qd


def fused(P, Q, k, V, U, UD, cfg):
    B = P.shape[0] // (k + 1)
    d = P.device
    drafts = torch.full((B * k,), -7, dtype=torch.int32, device=d)
    pd = (torch.full((B * (k + 1), 64), -7, dtype=torch.int32, device=d),
          torch.full((B * (k + 1), 64), 7.0, device=d), torch.full((B * (k + 1),), -7, dtype=torch.int32, device=d))
    qd = (torch.full((B * k, 64), -7, dtype=torch.int32, device=d), torch.full((B * k, 64), 7.0, device=d),
          torch.full((B * k,), -7, dtype=torch.int32, device=d))
    tok, n = vs.verify_windows(P[:, :V], Q[:, :V] if k else None, k, u_draft=UD if k else None, u=U,
                               drafts=drafts, p_dist=pd, q_dist=qd if k else None, **cfg)
    return tok, n, drafts, pd, qd


def same(a, b):
    a, b = host(a), host(b)
    return a.shape == b.shape and np.array_equal(a.view(np.uint8), b.view(np.uint8))


POLICIES = [
    CFG,
    dict(temperature=0.0, top_k=20, top_p=0.95, min_p=0.05),   # greedy policy
    dict(temperature=1.3, top_k=-1, top_p=1.0, min_p=0.0),     # absent top-k -> 20, no filters
    dict(temperature=0.7, top_k=0, top_p=0.5, min_p=0.2),      # 64-wide pool
    dict(temperature=2.0, top_k=5, top_p=0.3, min_p=0.5),
]

CONFIGS = [  # (seed, B, k, V, pad, policy)
    (100, 1, 3, 4096, 0, 0),
    (101, 257, 3, 4096, 0, 0),
    (102, 4096, 3, 4096, 0, 1),
    (103, 300, 1, 1000, 3, 2),
    (104, 64, 0, 4096, 0, 0),     # no drafts: the bonus draw alone
    (105, 100, 2, 64, 0, 3),      # the smallest vocabulary: the whole row is the pool
    (106, 33, 4, 2049, 0, 4),     # more rows than waves: waves take two rows
    (107, 20, 7, 4096, 8, 0),
    (108, 9, 15, 512, 0, 2),      # the most drafts
    (109, 500, 3, 4000, 96, 3),
    (110, 2000, 3, 128, 0, 1),
    (111, 1024, 3, 4096, 0, 0),   # the most windows of one launch
    (112, 1025, 3, 300, 4, 4),    # the fewest of two
]


@pytest.mark.parametrize("cfg", CONFIGS, ids=[f"B{c[1]}-k{c[2]}-V{c[3]}" for c in CONFIGS])
def test_matches_separate_calls(cfg):
    seed, B, k, V, pad, pol = cfg
    policy = POLICIES[pol]
    print(f"verify_windows: seed {seed} B {B} k {k} V {V} pad {pad} policy {policy}", flush=True)
    p, q, u, ud = case(seed, B, k, V, pad)
    P, Q, U, UD = dev(p), dev(q), dev(u), dev(ud)
    want = separate(P, Q, k, V, U, UD, policy)
    got = fused(P, Q, k, V, U, UD, policy)
    assert same(got[0], want[0]), "tokens"
    assert same(got[1], want[1]), "counts"
    if k:
        assert same(got[2], want[2]), "drafts"
        for a, b in zip(got[4], want[4]):
            assert same(a, b), "q distributions"
    for a, b in zip(got[3], want[3]):
        assert same(a, b), "p distributions"
    n = host(got[1])
    assert n.min() >= 1 and n.max() <= k + 1


def test_binding_allocated_outputs_and_a_side_stream():
    """Outputs left to the binding, the call on a non-default stream: the same bits."""
    p, q, u, ud = case(120, 777, 3, 4096)
    P, Q, U, UD = dev(p), dev(q), dev(u), dev(ud)
    want = fused(P, Q, 3, 4096, U, UD, CFG)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        tok, n = vs.verify_windows(P, Q, 3, u_draft=UD, u=U, **CFG)
    s.synchronize()
    assert same(tok, want[0]) and same(n, want[1])


@pytest.mark.parametrize("B,k,V", [(60, 3, 256), (6, 3, 4096), (20, 5, 1500)])
def test_stages_match_oracle(B, k, V):
    """Each stage against the oracle, fed what the previous stage produced."""
    p, q, u, ud = case(130 + V, B, k, V, special=False)
    P, Q, U, UD = dev(p), dev(q), dev(u), dev(ud)
    tok, n, drafts, pd, qd = (host(t) if isinstance(t, torch.Tensor) else tuple(host(x) for x in t)
                              for t in fused(P, Q, k, V, U, UD, CFG))
    pv, pi = topk_rows(p, 64)
    qv, qi = topk_rows(q, 64)
    for r in range(B * (k + 1)):
        ids, probs = policy_row(pv[r], pi[r], **CFG)
        L = int(pd[2][r])
        assert L == len(ids) and np.array_equal(pd[0][r, :L], ids), r
        assert ulp_diff_f32(pd[1][r, :L], probs).max() <= 1, r
        assert (pd[0][r, L:] == -1).all() and (pd[1][r, L:] == 0).all()
    for r in range(B * k):
        ids, probs = policy_row(qv[r], qi[r], **CFG)
        L = int(qd[2][r])
        assert L == len(ids) and np.array_equal(qd[0][r, :L], ids), r
        assert ulp_diff_f32(qd[1][r, :L], probs).max() <= 1, r
        # the draft is the oracle's draw from the GPU's q row
        assert drafts[r] == qd[0][r, draw(qd[1][r, :L], ud[r])], r
    for b in range(B):
        p_rows = [(pd[0][b * (k + 1) + i, :pd[2][b * (k + 1) + i]], pd[1][b * (k + 1) + i, :pd[2][b * (k + 1) + i]])
                  for i in range(k + 1)]
        q_rows = [(qd[0][b * k + i, :qd[2][b * k + i]], qd[1][b * k + i, :qd[2][b * k + i]]) for i in range(k)]
        want = accept_sampled(p_rows, q_rows, drafts[b * k:(b + 1) * k], u[b])
        assert list(tok[b, :n[b]]) == want, b
        assert (tok[b, n[b]:] == -1).all()


def test_first_token_follows_p():
    """200,000 windows over one set of rows: the first emitted token is
    distributed as p_0 (rejection sampling), whatever q proposes."""
    B, k, V = 200_000, 3, 256
    p1 = logits(140, (k + 1, V))
    q1 = correlated_logits(p1[:k], 0.5, 141)
    P = dev(p1).repeat(B, 1)
    Q = dev(q1).repeat(B, 1)
    U = dev(uniforms(142, (B, k + 1, 2)))
    UD = dev(uniforms(143, (B * k,)))
    tok, n = vs.verify_windows(P, Q, k, u_draft=UD, u=U, **CFG)
    first = host(tok)[:, 0]
    pv, pi = topk_rows(p1[:1], 64)
    ids, probs = policy_row(pv[0], pi[0], **CFG)
    assert np.isin(first, ids).all(), "every first token lies in p_0's support"
    assert chi2_pvalue(first, ids, probs) > 1e-4
    # the test has the power to tell p_0 from q_0, the draft's distribution
    qv, qi = topk_rows(q1[:1], 64)
    qids, qprobs = policy_row(qv[0], qi[0], **CFG)
    assert chi2_pvalue(first, qids, qprobs) < 1e-6


def test_full_batch_sampled_windows_against_oracle():
    """The bench's batch (16384 windows, k = 3, 4096 tokens, two launches):
    byte-identical to the separate calls, and 40 seeded windows against the
    oracle stage by stage."""
    B, k, V = 16384, 3, 4096
    print(f"verify_windows: full batch B {B} k {k} V {V}", flush=True)
    p, q, u, ud = case(150, B, k, V, special=False)
    P, Q, U, UD = dev(p), dev(q), dev(u), dev(ud)
    want = separate(P, Q, k, V, U, UD, CFG)
    got = fused(P, Q, k, V, U, UD, CFG)
    for a, b in ((got[0], want[0]), (got[1], want[1]), (got[2], want[2])):
        assert same(a, b)
    for a, b in zip(got[3] + got[4], want[3] + want[4]):
        assert same(a, b)
    tok, n, drafts = host(got[0]), host(got[1]), host(got[2])
    pd, qd = [tuple(host(t) for t in d) for d in (got[3], got[4])]
    for b in rng(151).choice(B, size=40, replace=False):
        p_rows, q_rows = [], []
        for rows, dist, logit_rows in ((p_rows, pd, p[b * (k + 1):(b + 1) * (k + 1)]),
                                       (q_rows, qd, q[b * k:(b + 1) * k])):
            base = b * (k + 1) if rows is p_rows else b * k
            vals, ids = topk_rows(logit_rows, 64)
            for i in range(len(logit_rows)):
                o_ids, o_probs = policy_row(vals[i], ids[i], **CFG)
                L = int(dist[2][base + i])
                assert L == len(o_ids) and np.array_equal(dist[0][base + i, :L], o_ids), (b, i)
                assert ulp_diff_f32(dist[1][base + i, :L], o_probs).max() <= 1, (b, i)
                rows.append((dist[0][base + i, :L], dist[1][base + i, :L]))
        for i in range(k):
            assert drafts[b * k + i] == q_rows[i][0][draw(q_rows[i][1], ud[b * k + i])], (b, i)
        assert list(tok[b, :n[b]]) == accept_sampled(p_rows, q_rows, drafts[b * k:(b + 1) * k], u[b]), b
