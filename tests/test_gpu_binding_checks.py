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
