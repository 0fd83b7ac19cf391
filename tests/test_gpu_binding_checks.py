"""The Python binding rejects malformed tensors before calling the C ABI.

Every call below must raise VerifySamplingError from the binding's own
checks (shape, stride, size, dtype, device); none of them reaches a kernel.
They need device tensors, hence the gpu mark, but launch nothing.
"""

from __future__ import annotations

import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def T():
    import torch

    import verify_sampling_amd as vs

    vs.library()
    dev = torch.device("cuda:0")

    def z(*shape, dtype=torch.float32):
        return torch.zeros(shape, dtype=dtype, device=dev)

    def i(*shape):
        return torch.zeros(shape, dtype=torch.int32, device=dev)

    return torch, vs, z, i


def raises(fn):
    import verify_sampling_amd as vs

    with pytest.raises(vs.VerifySamplingError):
        fn()


def test_gemv_rejects(T):
    torch, vs, z, i = T
    W = z(64, 32, dtype=torch.bfloat16)
    X = z(2, 32)
    raises(lambda: vs.verify_gemv_rows(W, z(2, 40)))                       # K mismatch
    raises(lambda: vs.verify_gemv_rows(W, X, z(2, 63)))                    # Y too narrow
    raises(lambda: vs.verify_gemv_rows(W, X, z(3, 64)))                    # Y rows
    raises(lambda: vs.verify_gemv_rows(W, X, z(2, 64, dtype=torch.float64)))
    raises(lambda: vs.verify_gemv_rows(W, z(2, 64)[:, ::2]))               # strided columns
    raises(lambda: vs.verify_gemv_rows(W, X.cpu()))                        # host tensor
    raises(lambda: vs.verify_gemv_rows(W, X, workspace=z(16)))             # float workspace
    raises(lambda: vs.verify_gemv_rows(W, X, workspace=i(4, 4).to(torch.uint8)[:, ::2]))
    raises(lambda: vs.verify_gemv_rows(W.float(), X))


def test_penalties_reject(T):
    torch, vs, z, i = T
    L = z(3, 100)
    kw = dict(window=4, repeat=1.1, presence=0.5, frequency=0.1)
    raises(lambda: vs.penalize_rows(L, i(2, 4), i(2), **kw))               # 2-D ctx
    raises(lambda: vs.penalize_rows(L, i(8)[::2], i(2), **kw))             # strided ctx
    raises(lambda: vs.penalize_rows(L, i(4), z(2), **kw))                  # float drafts
    raises(lambda: vs.penalize_rows(L, i(4), i(2), ids=i(3, 50), vocab=100, **kw))
    raises(lambda: vs.penalize_rows(z(3, 8), i(4), i(2), ids=i(3, 8), **kw))  # no vocab
    raises(lambda: vs.penalize_rows(L[:, ::2], i(4), i(2), **kw))
    raises(lambda: vs.penalize_tree_rows(z(4, 100), i(4), i(3), i(2), **kw))  # parent length
    raises(lambda: vs.penalize_tree_rows(z(3, 100), i(4), i(3), i(3), **kw))  # rows != nodes + 1
    raises(lambda: vs.penalize_tree_rows(z(4, 100), i(4), i(6)[::2], i(3), **kw))


def test_topk_rejects(T):
    torch, vs, z, i = T
    X = z(4, 1000)
    raises(lambda: vs.topk_rows(X, 16, z(3, 16), i(3, 16)))                # output rows
    raises(lambda: vs.topk_rows(X, 16, z(4, 8), i(4, 8)))                  # output width
    raises(lambda: vs.topk_rows(X, 16, z(4, 32), i(4, 16)))                # unequal strides
    raises(lambda: vs.topk_rows(X, 16, z(4, 16), z(4, 16)))                # float ids
    raises(lambda: vs.topk_rows(X[:, ::2], 16))
    raises(lambda: vs.topk_rows(X, 16, workspace=z(100)))


def test_policy_rejects(T):
    torch, vs, z, i = T
    V, I = z(4, 64), i(4, 64)
    cfg = dict(temperature=0.7, top_k=20, top_p=0.9, min_p=0.05)
    raises(lambda: vs.sample_policy_rows(V, i(4, 32), **cfg))              # ids shape
    raises(lambda: vs.sample_policy_rows(V, I, u=z(3), **cfg))             # u too short
    raises(lambda: vs.sample_policy_rows(V, I, u=i(4), **cfg))             # u dtype
    out = (i(4, 64), z(4, 64), i(3), None)
    raises(lambda: vs.sample_policy_rows(V, I, out=out, **cfg))            # dist_len too short
    out = (i(4, 64), z(4, 64), i(4), i(4))
    raises(lambda: vs.sample_policy_rows(V, I, out=out, **cfg))            # drawn without u
    out = (i(4, 64), z(4, 64), i(4), i(3))
    raises(lambda: vs.sample_policy_rows(V, I, u=z(4), out=out, **cfg))    # drawn too short
    out = (i(4, 32), z(4, 32), i(4), None)
    raises(lambda: vs.sample_policy_rows(V, I, out=out, **cfg))            # dist too narrow
    out = (i(4, 64), z(4, 80)[:, :64], i(4), None)
    raises(lambda: vs.sample_policy_rows(V, I, out=out, **cfg))            # unequal strides


def test_accept_rejects(T):
    torch, vs, z, i = T
    B, k = 2, 3
    d = i(B, k)
    p = (i(B * (k + 1), 8), z(B * (k + 1), 8), i(B * (k + 1)))
    q = (i(B * k, 8), z(B * k, 8), i(B * k))
    u = z(B, k + 1, 2)
    S = vs.ACCEPT_SAMPLED
    raises(lambda: vs.spec_accept_rows(S, d, p, q, u=z(B, k + 1, 1)))      # u too short
    raises(lambda: vs.spec_accept_rows(S, d, p, q))                        # u missing
    raises(lambda: vs.spec_accept_rows(S, d, p, None, u=u))                # q missing
    raises(lambda: vs.spec_accept_rows(S, d, (p[0][:-1], p[1][:-1], p[2]), q, u=u))  # p rows
    raises(lambda: vs.spec_accept_rows(S, d, (p[0], p[1], i(3)), q, u=u))  # p_len short
    raises(lambda: vs.spec_accept_rows(S, d, (p[0], z(B * (k + 1), 4), p[2]), q, u=u))
    raises(lambda: vs.spec_accept_rows(S, d, (p[0], None, p[2]), q, u=u))  # p_probs needed
    wide = i(B * (k + 1), 16)
    raises(lambda: vs.spec_accept_rows(S, d, (wide[:, :8], p[1], p[2]), q, u=u))  # row stride
    raises(lambda: vs.spec_accept_rows(S, d, p, (q[0], q[1], i(2)), u=u))  # q_len short
    raises(lambda: vs.spec_accept_rows(S, d, p, (q[0][:-1], q[1][:-1], q[2]), u=u))
    raises(lambda: vs.spec_accept_rows(S, d, (i(8, 65), z(8, 65), p[2]), q, u=u))  # > 64 wide
    raises(lambda: vs.spec_accept_rows(vs.ACCEPT_GREEDY_TREE, d, (p[0], None, None)))  # parent
    raises(lambda: vs.spec_accept_rows(vs.ACCEPT_GREEDY_TREE, d, (p[0], None, None),
                                       parent=i(B * k - 1)))
    raises(lambda: vs.spec_accept_rows(vs.ACCEPT_NAIVE, d, p))             # u missing
    raises(lambda: vs.spec_accept_rows(vs.ACCEPT_GREEDY, i(1, 6)[:, ::2], (p[0], None, None)))
    raises(lambda: vs.spec_accept_rows(S, d, p, q, u=u, out=(i(B, k), i(B))))  # tokens short
    raises(lambda: vs.spec_accept_rows(S, d, p, q, u=u, out=(i(B, k + 1), i(1))))
    raises(lambda: vs.spec_accept_rows(S, d, p, q, u=u, p_win_stride=-1))


def test_window_rejects(T):
    torch, vs, z, i = T
    R, V = 4, 1000
    L = z(R, V)
    ctx, dr = i(16), i(R - 1)
    qi, qv, u = i(R - 1, 8), z(R - 1, 8), z(R, 2)
    kw = dict(window=8, repeat=1.1, presence=0.5, frequency=0.1, temperature=0.7, top_k=20,
              top_p=0.9, min_p=0.05)
    ok = dict(q_ids=qi, q_vals=qv, u=u)
    raises(lambda: vs.verify_window(z(V), ctx, dr, **ok, **kw))                 # 1-D logits
    raises(lambda: vs.verify_window(L.double(), ctx, dr, **ok, **kw))           # dtype
    raises(lambda: vs.verify_window(L[:, ::2], ctx, dr, **ok, **kw))            # strided columns
    raises(lambda: vs.verify_window(L, ctx, i(R), **ok, **kw))                  # R - 1 drafts
    raises(lambda: vs.verify_window(L, i(4, 4), dr, **ok, **kw))                # 2-D history
    raises(lambda: vs.verify_window(L, ctx, z(R - 1), **ok, **kw))              # float drafts
    raises(lambda: vs.verify_window(L, ctx, dr, q_ids=qi, q_vals=qv, **kw))     # u missing
    raises(lambda: vs.verify_window(L, ctx, dr, q_ids=qi, q_vals=qv, u=z(2 * R - 1), **kw))
    raises(lambda: vs.verify_window(L, ctx, dr, q_ids=i(R - 1, 6), q_vals=qv, u=u, **kw))
    raises(lambda: vs.verify_window(L, ctx, dr, q_ids=i(R - 1, 65), q_vals=z(R - 1, 65), u=u, **kw))
    raises(lambda: vs.verify_window(L, ctx, dr, q_ids=qi, q_vals=z(R - 2, 8), u=u, **kw))
    raises(lambda: vs.verify_window(L, ctx, dr, **ok, workspace=z(64), **kw))  # float workspace
    good = dict(tokens=i(R), n=i(1), pool_vals=z(R, 64), pool_ids=i(R, 64),
                p=(i(R, 64), z(R, 64), i(R)), q=(i(R - 1, 8), z(R - 1, 8), i(R - 1)), q_pen=z(R - 1, 8))
    for key, bad in (("tokens", i(R - 1)), ("pool_vals", z(R, 32)), ("pool_ids", z(R, 64)),
                     ("p", (i(R, 64), z(R - 1, 64), i(R))), ("q", None),
                     ("q", (i(R - 1, 8), z(R - 1, 8), i(R - 2))), ("q_pen", z(R - 1, 4))):
        raises(lambda: vs.verify_window(L, ctx, dr, **ok, out=dict(good, **{key: bad}), **kw))


def test_tree_attention_rejects(T):
    torch, vs, z, i = T
    R, Hq, Hkv, D, n = 5, 4, 2, 128, 40
    q = z(R, Hq, D)
    kc = z(Hkv, n, D, dtype=torch.bfloat16)
    ks = z(Hkv, R, D, dtype=torch.bfloat16)
    par = i(R - 1)
    raises(lambda: vs.tree_attention_rows(z(R, Hq * D), kc, kc, n, ks, ks, par, scale=0.1))
    raises(lambda: vs.tree_attention_rows(q.double(), kc, kc, n, ks, ks, par, scale=0.1))
    raises(lambda: vs.tree_attention_rows(q, kc, kc, n, ks, z(Hkv, R + 1, D, dtype=torch.bfloat16),
                                          par, scale=0.1))                      # v_scr shape
    raises(lambda: vs.tree_attention_rows(q, z(Hkv, n, 64, dtype=torch.bfloat16), kc, n, ks, ks,
                                          par, scale=0.1))                      # cache head dim
    raises(lambda: vs.tree_attention_rows(q, kc.float(), kc, n, ks, ks, par, scale=0.1))
    raises(lambda: vs.tree_attention_rows(q, kc, kc, n, ks, ks, i(R - 2), scale=0.1))  # parent
    raises(lambda: vs.tree_attention_rows(q, kc, kc, n, ks, ks, None, scale=0.1))
    raises(lambda: vs.tree_attention_rows(q, kc, kc, n, ks, ks, par, scale=0.1,
                                          out=z(R, Hq, D - 1)))                 # out too small
    raises(lambda: vs.tree_attention_rows(q, kc, kc, n, ks, ks, par, scale=0.1,
                                          out=z(R, Hq, 2 * D)[:, :, :D]))       # strided out
    raises(lambda: vs.tree_attention_rows(q, kc, kc, n, ks, ks, par, scale=0.1, workspace=z(64)))
    raises(lambda: vs.tree_commit_kv(kc, kc, n - 3, z(Hkv, R, 64, dtype=torch.bfloat16),
                                     z(Hkv, R, 64, dtype=torch.bfloat16), i(2)))  # head dim
    raises(lambda: vs.tree_commit_kv(kc, kc, n - 3, ks, ks, z(2)))              # float path
    raises(lambda: vs.tree_commit_kv(kc, z(Hkv, n + 1, D, dtype=torch.bfloat16), n - 3, ks, ks,
                                     i(2)))                                     # cache shapes


def test_batched_windows_reject(T):
    torch, vs, z, i = T
    B, k, V = 4, 3, 256
    P, Q = z(B * (k + 1), V), z(B * k, V)
    U, UD = z(B, k + 1, 2), z(B * k)
    cfg = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)
    raises(lambda: vs.verify_windows(P[:-1], Q, k, u_draft=UD, u=U, **cfg))          # rows not B (k + 1)
    raises(lambda: vs.verify_windows(P, Q[:-1], k, u_draft=UD, u=U, **cfg))          # draft rows short
    raises(lambda: vs.verify_windows(P, z(B * k, V + 1), k, u_draft=UD, u=U, **cfg))  # vocab mismatch
    raises(lambda: vs.verify_windows(P, None, k, u_draft=UD, u=U, **cfg))            # q needed
    raises(lambda: vs.verify_windows(P, Q, k, u_draft=UD[:-1], u=U, **cfg))          # u_draft short
    raises(lambda: vs.verify_windows(P, Q, k, u_draft=UD, u=U[:-1], **cfg))          # u short
    raises(lambda: vs.verify_windows(P.double(), Q, k, u_draft=UD, u=U, **cfg))      # dtype
    raises(lambda: vs.verify_windows(P, Q, 16, u_draft=UD, u=U, **cfg))              # k > 15
    raises(lambda: vs.verify_windows(P, Q, k, u_draft=UD, u=U, drafts=i(B * k - 1), **cfg))
    raises(lambda: vs.verify_windows(P, Q, k, u_draft=UD, u=U, p_dist=(i(B * (k + 1), 32), z(B * (k + 1), 64),
                                                                     i(B * (k + 1))), **cfg))  # ids too small
    raises(lambda: vs.verify_windows(P, Q, k, u_draft=UD, u=U, q_dist=(i(B * k, 64), z(B * k, 64), i(B * k - 1)),
                                     **cfg))                                           # len too short
    raises(lambda: vs.verify_windows(P, Q, k, u_draft=UD, u=U, out=(i(B, k), i(B)), **cfg))  # tokens short
    raises(lambda: vs.verify_windows(P.cpu(), Q, k, u_draft=UD, u=U, **cfg))         # host tensor
