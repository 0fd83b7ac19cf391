"""verify_window (the acceptance stage in two launches) against the separate
calls it replaces, byte for byte, and against the oracle on seeded logits.

"Speculative decoding on RDNA": §04 (penalties of every verify row and of
the draft's candidates against H_i), §03 (pool, policy, rejection sampling),
§02 (greedy acceptance).  The separate sequence is penalize_rows (dense and
sparse), topk_rows at K = 64, sample_policy_rows for p and q and
spec_accept_rows; every output of the fused call (penalised logits, pools,
both distributions, the penalised candidates, tokens) must carry the same
bits.  Cases cover both chunk sizes of the pool selection and a single
chunk, ragged and unaligned rows, long and empty windows, one row and 64
rows, greedy mode, hard logits (ties across rank 64, +-inf, NaN, +-0, an
all-equal row) and histories with ids outside the vocabulary.
"""

import numpy as np
import pytest
import torch

import verify_sampling_amd as vs
from gpu_common import host, ulp_diff_f32
from oracle.accept import accept_sampled
from oracle.pipeline import acceptance_stage
from oracle.policy import policy_row
from synth import draft_candidates, logits, penalty_history, topk_planted_rows, uniforms

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
CFG = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)
PEN = dict(window=64, repeat=1.1, presence=1.5, frequency=0.2)


def make_case(seed, V, R, *, q_m=8, q_ld=None, ld=None, ctx_len=2080, planted=False, bad_ids=False,
              plateau=False):
    """Seeded window inputs: target logits [R][ld] (V valid), history, drafts,
    draft candidates [R-1][q_ld] (q_m valid), uniforms [R][2].  plateau: the
    first 2048 logits of every row equal 100.0 (so the history's hot tokens
    fall in chunks whose top K is selected by the exact path)."""
    k = R - 1
    ld = ld or V
    x = topk_planted_rows(seed, rows=R, vocab=V, K=64) if planted else logits(seed, (R, V))
    if plateau:
        x[:, :2048] = np.float32(100.0)
    lg = np.zeros((R, ld), dtype=np.float32)
    lg[:, :V] = x
    hot = np.unique(np.argsort(-np.nan_to_num(x, nan=-np.inf), axis=1)[:, :64])
    ctx = penalty_history(seed + 1, V, max(ctx_len - 32, 0), min(ctx_len, 32), hot)[:ctx_len]
    if bad_ids and ctx_len >= 8:
        ctx[[1, 5, ctx_len - 2]] = [-3, V + 5, V]   # never match a vocabulary entry
    q_ids = np.zeros((k, q_ld or q_m), dtype=np.int32)
    q_vals = np.zeros((k, q_ld or q_m), dtype=np.float32)
    drafts = np.zeros(k, dtype=np.int32)
    if k > 0:
        ids, vals = draft_candidates(seed + 2, np.nan_to_num(x[:k], nan=0.0, neginf=-1e30), q_m)
        q_ids[:, :q_m], q_vals[:, :q_m] = ids, vals
        pick = np.random.default_rng(seed + 3).integers(0, q_m, size=k)
        drafts = ids[np.arange(k), pick].astype(np.int32)
    u = uniforms(seed + 4, (R, 2))
    return lg, ctx, drafts, q_ids, q_vals, u


def to_dev(*arrays):
    return [torch.from_numpy(np.ascontiguousarray(a)).to(DEV) for a in arrays]


def separate(lg, ctx, drafts, q_ids, q_vals, u, V, q_m, pen, cfg):
    """The separate calls, on copies of the inputs."""
    L, C, D, U = to_dev(lg, ctx, drafts, u)
    Lv = L[:, :V]
    vs.penalize_rows(Lv, C, D, **pen)
    pv, pi = vs.topk_rows(Lv, 64)
    p = vs.sample_policy_rows(pv, pi, **cfg)[:3]
    k = len(drafts)
    sampled = cfg["temperature"] > 0
    out = dict(logits=L, pool_vals=pv, pool_ids=pi, p=p, q=None, q_pen=None)
    if sampled and k > 0:
        QI, QV = to_dev(q_ids[:, :q_m], q_vals[:, :q_m])
        vs.penalize_rows(QV, C, D, ids=QI, vocab=V, **pen)
        out["q"] = vs.sample_policy_rows(QV, QI, **cfg)[:3]
        out["q_pen"] = QV
    mode = vs.ACCEPT_SAMPLED if sampled else vs.ACCEPT_GREEDY
    tok, n = vs.spec_accept_rows(mode, D[None, :], p, out["q"], u=U[None] if sampled else None)
    out["tokens"], out["n"] = tok[0], n
    return out


def fused(lg, ctx, drafts, q_ids, q_vals, u, V, q_m, pen, cfg, workspace=None):
    L, C, D, U, QI, QV = to_dev(lg, ctx, drafts, u, q_ids, q_vals)
    QI0, QV0 = QI.clone(), QV.clone()
    out = vs.verify_window(L[:, :V], C, D, q_ids=QI[:, :q_m], q_vals=QV[:, :q_m], u=U,
                           workspace=workspace, **pen, **cfg)
    out["logits"] = L
    # the candidate inputs are not changed
    assert torch.equal(QI, QI0) and torch.equal(QV.view(torch.int32), QV0.view(torch.int32))
    return out


def bits(t):
    a = host(t)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_same(a, b, q_m):
    assert np.array_equal(bits(a["logits"]), bits(b["logits"])), "penalised logits"
    assert np.array_equal(bits(a["pool_vals"]), bits(b["pool_vals"])), "pool values"
    assert np.array_equal(bits(a["pool_ids"]), bits(b["pool_ids"])), "pool ids"
    for x, y, name in zip(a["p"], b["p"], ("p_ids", "p_probs", "p_len")):
        assert np.array_equal(bits(x), bits(y)), name
    if a["q"] is None:
        assert b["q"] is None
    else:
        for x, y, name in zip(a["q"], b["q"], ("q_ids", "q_probs", "q_len")):
            hx, hy = bits(x), bits(y)
            if hx.ndim == 2:
                hx, hy = hx[:, :q_m], hy[:, :q_m]
            assert np.array_equal(hx, hy), name
        assert np.array_equal(bits(a["q_pen"])[:, :q_m], bits(b["q_pen"])[:, :q_m]), "penalised candidates"
    n = int(host(a["n"])[0])
    assert n == int(host(b["n"])[0])
    assert np.array_equal(host(a["tokens"]), host(b["tokens"])), "tokens"
    assert 1 <= n <= len(host(a["tokens"]))


CASES = {
    # name: (seed, V, R, make_case options, penalty options, policy options)
    "lm_head_r4": (3000, 151936, 4, {}, {}, {}),
    "lm_head_r4_greedy": (3010, 151936, 4, {}, {}, dict(temperature=0.0)),
    "window_0": (3020, 151936, 4, {}, dict(window=0), {}),
    "long_window_hash_counts": (3030, 151936, 9, dict(ctx_len=6000), dict(window=4096), {}),
    "no_context": (3040, 151936, 5, dict(ctx_len=0), {}, {}),
    "one_row": (3050, 151936, 1, {}, {}, {}),
    "one_row_greedy": (3055, 151936, 1, {}, {}, dict(temperature=0.0)),
    "r25": (3060, 151936, 25, {}, {}, dict(top_k=0, top_p=1.0, min_p=0.0)),
    "r64_large_chunks": (3070, 151936, 64, {}, {}, {}),
    "one_chunk_v1000": (3080, 1000, 4, dict(q_m=5), {}, {}),
    "v4096_r8": (3090, 4096, 8, {}, dict(window=300), dict(temperature=1.3, top_k=64)),
    "unaligned_rows": (3100, 50257, 6, dict(ld=50260), {}, {}),
    "planted_hard_rows": (3110, 151936, 4, dict(planted=True, bad_ids=True), {}, {}),
    "q_stride": (3120, 32000, 4, dict(q_m=5, q_ld=12, bad_ids=True), dict(window=2000), {}),
    "negative_penalties": (3130, 151936, 4, {}, dict(presence=-0.5, frequency=-0.25, repeat=0.8), {}),
    # penalised history tokens lifted above a plateau: the chunk's exact path
    # reads the survivors' bits back from the row after the penalties' stores
    "plateau_lifted_history": (3140, 151936, 4, dict(plateau=True), dict(presence=-2.0, frequency=0.0, repeat=1.0), {}),
}


@pytest.mark.parametrize("name", list(CASES))
def test_fused_window_equals_separate_calls(name):
    seed, V, R, mk, pen_kw, cfg_kw = CASES[name]
    pen, cfg = dict(PEN, **pen_kw), dict(CFG, **cfg_kw)
    q_m = mk.get("q_m", 8)
    print(f"case {name}: V={V} R={R} pen={pen} cfg={cfg}", flush=True)
    lg, ctx, drafts, q_ids, q_vals, u = make_case(seed, V, R, **mk)
    a = fused(lg, ctx, drafts, q_ids, q_vals, u, V, q_m, pen, cfg)
    b = separate(lg, ctx, drafts, q_ids, q_vals, u, V, q_m, pen, cfg)
    assert_same(a, b, q_m)


def test_workspace_reuse_across_calls():
    """One workspace serves consecutive calls of different shapes (it holds
    nothing between calls)."""
    ws = torch.empty(vs.verify_window_workspace_bytes(64, 151936), dtype=torch.uint8, device=DEV)
    for seed, V, R in ((3200, 151936, 64), (3210, 151936, 4), (3220, 8192, 3)):
        lg, ctx, drafts, q_ids, q_vals, u = make_case(seed, V, R)
        a = fused(lg, ctx, drafts, q_ids, q_vals, u, V, 8, PEN, CFG, workspace=ws)
        b = separate(lg, ctx, drafts, q_ids, q_vals, u, V, 8, PEN, CFG)
        assert_same(a, b, 8)


@pytest.mark.parametrize("seed", [3300, 3310])
def test_fused_window_against_oracle(seed):
    """The oracle's stages on the same seeded logits: penalised rows and pools
    bit for bit; policy ids exact and probabilities within 1 ulp; tokens
    equal to the oracle's acceptance of the GPU's own distributions."""
    V, R = 151936, 4
    lg, ctx, drafts, q_ids, q_vals, u = make_case(seed, V, R, bad_ids=True)
    got = fused(lg, ctx, drafts, q_ids, q_vals, u, V, 8, PEN, CFG)
    want = acceptance_stage(lg, ctx, drafts, u, q_ids=q_ids, q_vals=q_vals, **PEN, **CFG)
    assert np.array_equal(bits(got["logits"]), want["penalized"].view(np.uint32))
    assert np.array_equal(host(got["pool_ids"]), want["pool_ids"])
    assert np.array_equal(bits(got["pool_vals"]), want["pool_vals"].view(np.uint32))
    assert np.array_equal(bits(got["q_pen"]), want["q_penalized"].view(np.uint32))

    def rows(dist, oracle_rows):
        ids, probs, ln = (host(t) for t in dist)
        out = []
        for i, (oi, op) in enumerate(oracle_rows):
            assert ln[i] == len(oi) and np.array_equal(ids[i, :ln[i]], oi), i
            assert (ulp_diff_f32(probs[i, :ln[i]], op) <= 1).all(), i
            out.append((ids[i, :ln[i]], probs[i, :ln[i]]))
        return out

    p_rows = rows(got["p"], want["p_rows"])
    q_rows = rows(got["q"], want["q_rows"])
    n = int(host(got["n"])[0])
    assert list(host(got["tokens"])[:n]) == accept_sampled(p_rows, q_rows, drafts, u)


def test_q_policy_matches_oracle_policy_rows():
    """The draft side alone: the penalised candidates and their distribution
    against the oracle (q rows with a stride and fewer candidates)."""
    V, R, q_m = 32000, 6, 5
    lg, ctx, drafts, q_ids, q_vals, u = make_case(3400, V, R, q_m=q_m, q_ld=7)
    got = fused(lg, ctx, drafts, q_ids, q_vals, u, V, q_m, PEN, CFG)
    want = acceptance_stage(lg[:, :V], ctx, drafts, u, q_ids=q_ids[:, :q_m], q_vals=q_vals[:, :q_m],
                            **PEN, **CFG)
    assert np.array_equal(bits(got["q_pen"])[:, :q_m], want["q_penalized"].view(np.uint32))
    ids, probs, ln = (host(t) for t in got["q"])
    for i in range(R - 1):
        oi, op = policy_row(want["q_penalized"][i], q_ids[i, :q_m], **CFG)
        assert ln[i] == len(oi) and np.array_equal(ids[i, :ln[i]], oi)
        assert (ulp_diff_f32(probs[i, :ln[i]], op) <= 1).all()


def random_config(seed):
    g = np.random.default_rng(seed)
    V = int(g.choice([64, 100, 1024, 1500, 4096, 32000, 50257, 151936]))
    R = int(g.integers(1, 65))
    q_m = int(g.integers(1, 17))
    mk = dict(q_m=q_m, q_ld=q_m + int(g.integers(0, 4)), ld=V + int(g.choice([0, 0, 1, 3, 8])),
              ctx_len=int(g.choice([0, 1, 5, 64, 300, 5000])), bad_ids=bool(g.integers(0, 2)),
              planted=bool(V >= 1024 and g.integers(0, 4) == 0))
    pen = dict(window=int(g.choice([0, 1, 7, 64, 200, 4096])), repeat=float(g.choice([0.5, 1.0, 1.3])),
               presence=float(g.uniform(-1, 2)), frequency=float(g.uniform(-0.5, 0.5)))
    cfg = dict(temperature=float(g.choice([0.0, 0.3, 0.7, 1.0, 2.5])), top_k=int(g.choice([-1, 0, 1, 5, 20, 64])),
               top_p=float(g.choice([0.1, 0.9, 1.0])), min_p=float(g.choice([0.0, 0.05, 0.5])))
    return V, R, mk, pen, cfg


@pytest.mark.parametrize("seed", range(3500, 3524))
def test_fused_window_random_configurations(seed):
    """Seeded random windows (vocabulary, rows up to 64, row and candidate
    strides, context and window lengths, penalty signs, every policy
    setting, greedy and sampled): the fused call equals the separate calls
    byte for byte."""
    V, R, mk, pen, cfg = random_config(seed)
    print(f"seed {seed}: V={V} R={R} {mk} {pen} {cfg}", flush=True)
    lg, ctx, drafts, q_ids, q_vals, u = make_case(seed, V, R, **mk)
    a = fused(lg, ctx, drafts, q_ids, q_vals, u, V, mk["q_m"], pen, cfg)
    b = separate(lg, ctx, drafts, q_ids, q_vals, u, V, mk["q_m"], pen, cfg)
    assert_same(a, b, mk["q_m"])
