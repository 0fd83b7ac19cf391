"""HIP-graph capture of a verify window through the C ABI.

Every entry point validates on the host and then only enqueues kernels on
the caller's stream: no allocation, no memset, no host synchronisation.  A
window captured once as a graph therefore replays with the same bits as the
same calls made eagerly.  The window here takes the paths that use a
workspace:
  * the projection's split-K path (4096 x 12288 at 12 rows, partial sums plus
    the in-order partition sum);
  * the top-K's multi-chunk path (vocab 32768, a merge over the chunks);
  * penalties on the logits and on the draft's candidates;
  * the policy for p and q with a draw;
  * speculative rejection sampling ("Speculative decoding on RDNA", §03).
Before each replay the inputs are overwritten and the window runs eagerly on
them; every replay must equal that eager result bit for bit.
"""

import numpy as np
import pytest
import torch

import verify_sampling_amd as vs
from gpu_common import DEV, host
from synth import draft_candidates, logits, penalty_history, torch_bf16_weights, uniforms

pytestmark = pytest.mark.gpu
CFG = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)
PEN = dict(window=64, repeat=1.1, presence=1.5, frequency=0.2)
K_DRAFT = 3
VOCAB, HIDDEN = 32768, 2048


def new_inputs(seed):
    g = np.random.default_rng(seed)
    x1 = g.standard_normal((12, 12288), dtype=np.float32)
    x2 = g.standard_normal((K_DRAFT + 1, HIDDEN), dtype=np.float32)
    q_ids, q_vals = draft_candidates(seed + 1, logits(seed + 2, (K_DRAFT, VOCAB)), 8)
    drafts = q_ids[:, 0].copy()
    ctx = penalty_history(seed + 3, VOCAB, 512, 16, q_ids.reshape(-1))
    u = uniforms(seed + 4, (1, K_DRAFT + 1, 2))
    u_pol = uniforms(seed + 5, (K_DRAFT + 1,))
    return dict(x1=x1, x2=x2, q_ids=q_ids, q_vals=q_vals, drafts=drafts, ctx=ctx, u=u,
                u_pol=u_pol)


@pytest.fixture(scope="module")
def window_state():
    W1 = torch_bf16_weights((4096, 12288), 2600, DEV)
    W2 = torch_bf16_weights((VOCAB, HIDDEN), 2601, DEV)
    first = new_inputs(2602)
    bufs = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in first.items()}
    return W1, W2, bufs


def window(W1, W2, b):
    """One verify window on the current stream; returns every output."""
    ws1 = torch.empty(vs.verify_gemv_rows_workspace_bytes(4096, 12288, 12), dtype=torch.uint8,
                      device=DEV)
    Y1 = vs.verify_gemv_rows(W1, b["x1"], workspace=ws1)
    L = vs.verify_gemv_rows(W2, b["x2"])
    raw = L.clone()
    vs.penalize_rows(L, b["ctx"], b["drafts"], **PEN)
    pv, pi = vs.topk_rows(L, 64)
    p = vs.sample_policy_rows(pv, pi, **CFG, u=b["u_pol"])
    qv = b["q_vals"].clone()
    vs.penalize_rows(qv, b["ctx"], b["drafts"], ids=b["q_ids"], vocab=VOCAB, **PEN)
    q = vs.sample_policy_rows(qv, b["q_ids"], **CFG)
    tok, n = vs.spec_accept_rows(vs.ACCEPT_SAMPLED, b["drafts"][None, :], p[:3], q[:3], u=b["u"])
    return dict(Y1=Y1, raw=raw, L=L, pv=pv, pi=pi, p_ids=p[0], p_probs=p[1], p_len=p[2],
                p_drawn=p[3], qv=qv, q_ids=q[0], q_probs=q[1], q_len=q[2], tok=tok, n=n)


def test_window_replays_equal_eager(window_state):
    W1, W2, bufs = window_state
    assert vs.verify_gemv_rows_workspace_bytes(4096, 12288, 12) > 0  # the split-K path
    assert vs.topk_rows_workspace_bytes(K_DRAFT + 1, VOCAB, 64) > 0  # the multi-chunk path

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        window(W1, W2, bufs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = window(W1, W2, bufs)

    seen = []
    for rep, seed in enumerate([2710, 2720, 2730]):
        for k, v in new_inputs(seed).items():
            bufs[k].copy_(torch.from_numpy(np.ascontiguousarray(v)))
        eager = {k: host(v) for k, v in window(W1, W2, bufs).items()}
        graph.replay()
        got = {k: host(v) for k, v in captured.items()}
        for k in eager:
            a, b = eager[k], got[k]
            assert a.shape == b.shape, (rep, k)
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (rep, k)
        assert 1 <= int(eager["n"][0]) <= K_DRAFT + 1
        seen.append(got["Y1"].tobytes() + got["pi"].tobytes())
    assert len(set(seen)) == len(seen)  # each replay computed on its own inputs
