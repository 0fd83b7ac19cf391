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


def fused_window(W2, b, t):
    """The LM-head projection, verify_window and tree attention with the
    commit of a branch, on the current stream."""
    L = vs.verify_gemv_rows(W2, b["x2"])
    raw = L.clone()
    out = vs.verify_window(L, b["ctx"], b["drafts"], q_ids=b["q_ids"], q_vals=b["q_vals"],
                           u=b["u"][0], **PEN, **CFG)
    att = vs.tree_attention_rows(t["q"], t["kc"], t["vc"], 200, t["ks"], t["vs"], t["parent"],
                                 scale=0.0883883)
    kc, vc = t["kc"].clone(), t["vc"].clone()
    vs.tree_commit_kv(kc, vc, 200, t["ks"], t["vs"], t["path"])
    res = dict(raw=raw, L=L, att=att, kc=kc, vc=vc, tokens=out["tokens"], n=out["n"],
               pool_vals=out["pool_vals"], pool_ids=out["pool_ids"], q_pen=out["q_pen"])
    for name, tup in (("p", out["p"]), ("q", out["q"])):
        for j, tt in enumerate(tup):
            res[f"{name}{j}"] = tt
    return res


def tree_inputs(seed):
    g = np.random.default_rng(seed)
    R, Hq, Hkv, D, L = 9, 8, 2, 128, 256
    f = lambda shape: torch.from_numpy(g.standard_normal(shape, dtype=np.float32)).to(DEV)
    return dict(q=f((R, Hq, D)), kc=f((Hkv, L, D)).to(torch.bfloat16), vc=f((Hkv, L, D)).to(torch.bfloat16),
                ks=f((Hkv, R, D)).to(torch.bfloat16), vs=f((Hkv, R, D)).to(torch.bfloat16))


def test_fused_window_and_tree_attention_replay_equal_eager(window_state):
    """verify_window (its multi-chunk select and one-workgroup finish) and
    tree attention (split and merge kernels) with the commit, captured once
    and replayed on fresh inputs: every replay equals the eager run bit for
    bit."""
    _, W2, bufs = window_state
    t = tree_inputs(2800)
    t["parent"] = torch.tensor([-1, 0, 1, -1, 3, 4, 0, 6], dtype=torch.int32, device=DEV)
    t["path"] = torch.tensor([0, 4, 5, 6], dtype=torch.int32, device=DEV)
    assert vs.verify_window_workspace_bytes(K_DRAFT + 1, VOCAB) > 0

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fused_window(W2, bufs, t)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        captured = fused_window(W2, bufs, t)

    for rep, seed in enumerate([2810, 2820, 2830]):
        for k, v in new_inputs(seed).items():
            bufs[k].copy_(torch.from_numpy(np.ascontiguousarray(v)))
        for k, v in tree_inputs(seed + 1).items():
            t[k].copy_(v)
        eager = {k: host(v) for k, v in fused_window(W2, bufs, t).items()}
        graph.replay()
        got = {k: host(v) for k, v in captured.items()}
        for k in eager:
            assert np.array_equal(eager[k].view(np.uint8), got[k].view(np.uint8)), (rep, k)
        assert 1 <= int(eager["n"][0]) <= K_DRAFT + 1


def test_tree_window_replays_equal_eager():
    """verify_tree_window on a 2 x 4 tree (9 rows of 151936 logits: two
    finish workgroups, so the arrival counter too) captured once and
    replayed on fresh inputs: every replay equals the eager run bit for bit."""
    from synth import tree_window

    V = 151936
    pen = dict(window=64, repeat=1.1, presence=1.5, frequency=0.2)
    cfg = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)

    def inputs(seed):
        lg, ctx, tokens, parent, u = tree_window(seed, V, branches=2, depth=4)
        return dict(logits=lg, ctx=ctx, tokens=tokens, parent=parent, u=u)

    bufs = {k: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for k, v in inputs(2900).items()}
    work = torch.empty_like(bufs["logits"])
    R = work.shape[0]
    ws = torch.empty(vs.verify_window_workspace_bytes(R, V), dtype=torch.uint8, device=DEV)
    out = dict(tokens=torch.empty((R,), dtype=torch.int32, device=DEV),
               n=torch.empty((1,), dtype=torch.int32, device=DEV),
               pool_vals=torch.empty((R, 64), device=DEV),
               pool_ids=torch.empty((R, 64), dtype=torch.int32, device=DEV),
               p=(torch.empty((R, 64), dtype=torch.int32, device=DEV), torch.empty((R, 64), device=DEV),
                  torch.empty((R,), dtype=torch.int32, device=DEV)))

    def run():
        work.copy_(bufs["logits"])  # penalised in place: every run starts from the inputs
        vs.verify_tree_window(work, bufs["ctx"], bufs["tokens"], bufs["parent"], u=bufs["u"], out=out,
                              workspace=ws, **pen, **cfg)

    def snapshot():
        flat = dict(work=work, tokens=out["tokens"], n=out["n"], pool_vals=out["pool_vals"],
                    pool_ids=out["pool_ids"], p_ids=out["p"][0], p_probs=out["p"][1], p_len=out["p"][2])
        return {k: host(v) for k, v in flat.items()}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()

    for rep, seed in enumerate([2910, 2920, 2930]):
        for k, v in inputs(seed).items():
            bufs[k].copy_(torch.from_numpy(np.ascontiguousarray(v)))
        run()
        eager = snapshot()
        graph.replay()
        got = snapshot()
        for k in eager:
            assert np.array_equal(eager[k].view(np.uint8), got[k].view(np.uint8)), (rep, k)
        assert 1 <= int(eager["n"][0]) <= R


@pytest.mark.parametrize("B", [64, 2048])
def test_batched_windows_replay_equal_eager(B):
    """verify_windows (one launch at 64 windows, two at 2048) captured once
    and replayed on fresh target and draft rows and uniforms: every replay
    equals the eager run bit for bit."""
    k, V = 3, 4096
    cfg = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)

    def inputs(seed):
        return dict(p=logits(seed, (B * (k + 1), V)), q=logits(seed + 1, (B * k, V)),
                    u=uniforms(seed + 2, (B, k + 1, 2)), ud=uniforms(seed + 3, (B * k,)))

    bufs = {n: torch.from_numpy(np.ascontiguousarray(v)).to(DEV) for n, v in inputs(3000).items()}
    outs = dict(drafts=torch.empty((B * k,), dtype=torch.int32, device=DEV),
                p=(torch.empty((B * (k + 1), 64), dtype=torch.int32, device=DEV),
                   torch.empty((B * (k + 1), 64), device=DEV),
                   torch.empty((B * (k + 1),), dtype=torch.int32, device=DEV)),
                q=(torch.empty((B * k, 64), dtype=torch.int32, device=DEV), torch.empty((B * k, 64), device=DEV),
                   torch.empty((B * k,), dtype=torch.int32, device=DEV)),
                out=(torch.empty((B, k + 1), dtype=torch.int32, device=DEV),
                     torch.empty((B,), dtype=torch.int32, device=DEV)))

    def run():
        vs.verify_windows(bufs["p"], bufs["q"], k, u_draft=bufs["ud"], u=bufs["u"], drafts=outs["drafts"],
                          p_dist=outs["p"], q_dist=outs["q"], out=outs["out"], **cfg)

    def snapshot():
        flat = [outs["drafts"], *outs["p"], *outs["q"], *outs["out"]]
        return [host(t) for t in flat]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run()

    for rep, seed in enumerate([3010, 3020, 3030]):
        for n, v in inputs(seed).items():
            bufs[n].copy_(torch.from_numpy(np.ascontiguousarray(v)))
        run()
        eager = snapshot()
        graph.replay()
        got = snapshot()
        for i, (a, b) in enumerate(zip(eager, got)):
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), (rep, i)
        assert eager[-1].min() >= 1
