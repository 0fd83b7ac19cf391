"""Benchmark of one speculative-decoding verify window on one MI355X.

A step is one verify pass over the whole hot path:
  * the projections of a 36-layer 8B-class decoder stack (per layer: q|k|v,
    o, gate|up and down, bf16 weights stored fused where the projections
    share an input) for R = k + 1 = 4 rows,
  * the 151936 x 4096 LM head for the same rows,
  * the acceptance stage: penalties on the R target rows (window 64,
    repeat 1.1, presence 1.5, frequency 0.2) and on the draft's 8
    re-scored candidates per draft row, the top-64 pool, the sampler policy
    (temperature 0.7, top-k 20, top-p 0.95, min-p 0.05) for p and q, and
    speculative rejection acceptance with the bonus draw, all in one
    verify_window call (two launches; the seven separate calls it replaces
    are timed beside it).
Inputs (synthetic, seeded, N(0, 0.02) bf16 weights, N(0, 1) activations)
are resident in HBM before timing starts.  `value` is the algorithmic bytes
of the pass divided by the step time.

Also reported: time per pass of the projections for every R from 1 to 24
(the knee), the roofline of the projection kernel, batched sampling rows/s
(vocab 4096, k = 3, 16384 windows each with its own rows), and the oracle
on the host cores as the CPU baseline.

    python bench.py [--gpus 1] [--steps 20] [--warmup 3] [--rows 4]
                    [--no-sweep] [--no-cpu-baseline] [--graph]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
CALIB_BYTES = 1 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemv_rows_traffic_r{R}.md")
KERNEL_SOURCE = os.path.join(ROOT, "verify_sampling_amd", "csrc", "gemv_rows.hip")


def measured_traffic(R):
    """HBM bytes per projection launch from the committed counter summary.

    None unless the summary was taken at this R from the current kernel
    source (its sha256 is recorded in the summary).
    """
    import hashlib
    import re

    try:
        text = open(TRAFFIC_FILE.format(R=R)).read()
        src = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    m = re.search(r"kernel_source_sha256:\s*([0-9a-f]{64})", text)
    r = re.search(r"rows:\s*(\d+)", text)
    b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not (m and r and b) or m.group(1) != src or int(r.group(1)) != R:
        return None
    return float(b.group(1))
CFG = dict(temperature=0.7, top_k=20, top_p=0.95, min_p=0.05)
PEN = dict(window=64, repeat=1.1, presence=1.5, frequency=0.2)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--rows", type=int, default=4, help="verify rows R = k + 1")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sampling", action="store_true")
    ap.add_argument("--projections-only", action="store_true",
                    help="time the step and the projection pass, then stop (profiler runs: "
                         "the other legs add thousands of dispatches)")
    ap.add_argument("--graph", action="store_true", help="replay the step as a HIP graph")
    ap.add_argument("--layers", type=int, default=36)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one 1 GiB device copy first (for scaling HBM traffic counters)")
    ap.add_argument("--family-sweep", action="store_true",
                    help="only time verify_gemv_rows per matrix on three model sizes "
                         "(hidden 2560, 4096, 5120) for R = 1..24 and print that as the JSON line")
    return ap.parse_args()


class VerifyPass:
    """All inputs of one verify window, resident on the GPU."""

    def __init__(self, torch, vs, synth, layers, rmax, dev):
        self.torch, self.vs = torch, vs
        self.dev = dev
        self.mats = []  # (W, X[rmax][K], Y[rmax][N])
        seed = 5000
        g = torch.Generator(device=dev)
        for layer in range(layers):
            for name, (N, K) in synth.LAYER_SHAPES_FUSED.items():
                W = synth.torch_bf16_weights((N, K), seed, dev)
                g.manual_seed(seed + 1)
                X = torch.randn((rmax, K), generator=g, device=dev, dtype=torch.float32)
                Y = torch.empty((rmax, N), device=dev, dtype=torch.float32)
                self.mats.append((W, X, Y))
                seed += 2
        N, K = synth.LM_HEAD_SHAPE
        self.head = synth.torch_bf16_weights((N, K), seed, dev)
        g.manual_seed(seed + 1)
        self.head_x = torch.randn((rmax, K), generator=g, device=dev, dtype=torch.float32)
        self.logits = torch.empty((rmax, N), device=dev, dtype=torch.float32)
        self.vocab = N
        self._arg_cache = {}
        torch.cuda.synchronize()

    def bytes_projections(self, R):
        tot = 0
        for W, X, Y in self.mats:
            N, K = W.shape
            tot += 2 * N * K + 4 * R * (K + N)
        N, K = self.head.shape
        tot += 2 * N * K + 4 * R * (K + N)
        return tot

    def n_launches(self):
        return len(self.mats) + 1

    def _args(self, R):
        """C-ABI arguments of every projection launch at R rows (pointers cached).

        The launches run in order on one stream, so they share one workspace
        sized for the largest of them.
        """
        if R not in self._arg_cache:
            mats = self.mats + [(self.head, self.head_x, self.logits)]
            nbytes = max(self.vs.verify_gemv_rows_workspace_bytes(W.shape[0], W.shape[1], R)
                         for W, _, _ in mats)
            ws = self.torch.empty(max(nbytes, 16), dtype=self.torch.uint8, device=self.dev)
            out = []
            for W, X, Y in mats:
                N, K = W.shape
                out.append((W.data_ptr(), K, N, K, X.data_ptr(), K, R, Y.data_ptr(), N,
                            ws.data_ptr(), nbytes))
            self._arg_cache[R] = (out, ws)
        return self._arg_cache[R][0]

    def projections(self, R):
        """The R-row projections of the stack and the LM head, in pass order."""
        fn = self.vs.library().verify_gemv_rows
        stream = self.torch.cuda.current_stream().cuda_stream
        for a in self._args(R):
            st = fn(*a, stream)
            if st != 0:
                raise RuntimeError(f"verify_gemv_rows failed with status {st}")

    def setup_acceptance(self, synth, R):
        """History, draft candidates and drafts for a window of k = R - 1 drafts."""
        torch, vs, dev = self.torch, self.vs, self.dev
        k = R - 1
        self.R, self.k = R, k
        self.projections(R)
        torch.cuda.synchronize()
        lg = self.logits[:R].cpu().numpy()
        hot = np.unique(np.argsort(-lg, axis=1)[:, :64])
        ctx = synth.penalty_history(6001, self.vocab, 2048, 32, hot)
        q_ids, q_vals = synth.draft_candidates(6002, lg[:k], 8)
        self.ctx = torch.from_numpy(ctx).to(dev)
        self.q_ids = torch.from_numpy(q_ids).to(dev)
        self.q_raw = torch.from_numpy(q_vals).to(dev)
        self.q_vals = self.q_raw.clone()
        self.u = torch.from_numpy(synth.uniforms(6003, (1, R, 2))).to(dev)
        ud = torch.from_numpy(synth.uniforms(6004, (k, 1))).to(dev)
        # the drafter's own sequential draws: d_i ~ q_i penalised by H_i
        drafts = torch.zeros((k,), dtype=torch.int32, device=dev)
        for i in range(k):
            # row i's history holds drafts[0, i): penalise a copy of all rows, keep row i
            allq = self.q_raw.clone()
            vs.penalize_rows(allq, self.ctx, drafts[:i].contiguous(), ids=self.q_ids,
                             vocab=self.vocab, **PEN)
            _, _, _, drawn = vs.sample_policy_rows(allq[i:i + 1].contiguous(),
                                                   self.q_ids[i:i + 1].contiguous(),
                                                   u=ud[i], **CFG)
            drafts[i] = drawn[0]
        self.drafts = drafts
        # one workspace for the separate top-K call and for verify_window
        # (which also needs an arrival counter above 8 rows)
        self.ws = torch.empty(max(vs.topk_rows_workspace_bytes(R, self.vocab, 64),
                                  vs.verify_window_workspace_bytes(R, self.vocab)),
                              dtype=torch.uint8, device=dev)
        self.pool_v = torch.empty((R, 64), device=dev, dtype=torch.float32)
        self.pool_i = torch.empty((R, 64), device=dev, dtype=torch.int32)
        self.p_out = (torch.empty((R, 64), dtype=torch.int32, device=dev),
                      torch.empty((R, 64), dtype=torch.float32, device=dev),
                      torch.empty((R,), dtype=torch.int32, device=dev), None)
        self.q_out = (torch.empty((k, 8), dtype=torch.int32, device=dev),
                      torch.empty((k, 8), dtype=torch.float32, device=dev),
                      torch.empty((k,), dtype=torch.int32, device=dev), None)
        self.acc_out = (torch.empty((1, R), dtype=torch.int32, device=dev),
                        torch.empty((1,), dtype=torch.int32, device=dev))
        self._acc_calls = self._acceptance_calls()
        self.win_out = dict(tokens=torch.empty((R,), dtype=torch.int32, device=dev),
                            n=torch.empty((1,), dtype=torch.int32, device=dev),
                            pool_vals=torch.empty((R, 64), dtype=torch.float32, device=dev),
                            pool_ids=torch.empty((R, 64), dtype=torch.int32, device=dev),
                            p=tuple(torch.empty_like(t) for t in self.p_out[:3]),
                            q=tuple(torch.empty_like(t) for t in self.q_out[:3]),
                            q_pen=torch.empty_like(self.q_raw))
        self._win_args = self._fused_args()
        torch.cuda.synchronize()
        # the cached C-ABI calls give the binding's result (penalties work in
        # place, so the logits are computed afresh for each), and the fused
        # window gives the separate calls' bits
        self.projections(R)
        self.acceptance_binding()
        ref = [t.clone() for t in self.acc_out]
        ref_pen = self.logits[:R].clone()
        self.projections(R)
        self.acceptance_separate()
        torch.cuda.synchronize()
        if not all(torch.equal(a, b) for a, b in zip(ref, self.acc_out)):
            raise RuntimeError("cached acceptance calls disagree with the binding")
        self.projections(R)
        self.acceptance()
        torch.cuda.synchronize()
        w = self.win_out
        same = (torch.equal(w["tokens"], ref[0][0]) and torch.equal(w["n"], ref[1]) and
                torch.equal(self.logits[:R].view(torch.int32), ref_pen.view(torch.int32)) and
                torch.equal(w["pool_ids"], self.pool_i) and
                all(torch.equal(a.view(torch.int32), b.view(torch.int32))
                    for a, b in zip(w["p"] + w["q"], self.p_out[:3] + self.q_out[:3])))
        if not same:
            raise RuntimeError("verify_window disagrees with the separate calls")

    def acceptance_binding(self):
        """The acceptance stage through the Python binding (argument checks on every call)."""
        vs, R, k = self.vs, self.R, self.k
        L = self.logits[:R]
        vs.penalize_rows(L, self.ctx, self.drafts, **PEN)
        vs.topk_rows(L, 64, self.pool_v, self.pool_i, self.ws)
        p = vs.sample_policy_rows(self.pool_v, self.pool_i, out=self.p_out, **CFG)
        self.q_vals.copy_(self.q_raw)  # the draft's re-scored candidates for this window
        vs.penalize_rows(self.q_vals, self.ctx, self.drafts, ids=self.q_ids, vocab=self.vocab, **PEN)
        q = vs.sample_policy_rows(self.q_vals, self.q_ids, out=self.q_out, **CFG)
        vs.spec_accept_rows(vs.ACCEPT_SAMPLED, self.drafts[None, :], p[:3], q[:3], u=self.u,
                            out=self.acc_out)

    def _acceptance_calls(self):
        """The same launches as C-ABI calls with their arguments prepared once
        (all but the stream, taken at call time so that graph capture sees
        them), so that the timed stage is the GPU's work rather than argument
        marshalling.  (Running the draft side on a second stream, joined with
        events, made the stage slower: 88 against 44 us.)"""
        vs, R, k, V = self.vs, self.R, self.k, self.vocab
        lib = vs.library()
        L = self.logits[:R]
        pen = (PEN["window"], PEN["repeat"], PEN["presence"], PEN["frequency"])
        cfg = (CFG["temperature"], CFG["top_k"], CFG["top_p"], CFG["min_p"])
        ctx, n_ctx, dr = self.ctx.data_ptr(), int(self.ctx.numel()), self.drafts.data_ptr()
        nws = int(self.ws.numel())
        p_ids, p_probs, p_len = (t.data_ptr() for t in self.p_out[:3])
        q_ids, q_probs, q_len = (t.data_ptr() for t in self.q_out[:3])
        return [
            (lib.penalize_rows, (L.data_ptr(), None, L.stride(0), R, V, V, ctx, n_ctx, dr, k, *pen)),
            (lib.topk_rows, (L.data_ptr(), L.stride(0), R, V, 64, self.pool_v.data_ptr(),
                             self.pool_i.data_ptr(), 64, self.ws.data_ptr() if nws else None, nws)),
            (lib.sample_policy_rows, (self.pool_v.data_ptr(), self.pool_i.data_ptr(), 64, R, 64, *cfg,
                                      p_ids, p_probs, p_len, 64, None, None)),
            (None, None),  # the draft's re-scored candidates for this window
            (lib.penalize_rows, (self.q_vals.data_ptr(), self.q_ids.data_ptr(), 8, k, 8, V, ctx, n_ctx,
                                 dr, k, *pen)),
            (lib.sample_policy_rows, (self.q_vals.data_ptr(), self.q_ids.data_ptr(), 8, k, 8, *cfg,
                                      q_ids, q_probs, q_len, 8, None, None)),
            (lib.spec_accept_rows, (vs.ACCEPT_SAMPLED, 1, k, p_ids, p_probs, p_len, 64, k + 1,
                                    q_ids, q_probs, q_len, 8, k, dr, None, self.u.data_ptr(),
                                    self.acc_out[0].data_ptr(), self.acc_out[1].data_ptr())),
        ]

    def _fused_args(self):
        """verify_window's arguments, prepared once (the stream is taken at call time)."""
        vs, R, k, V = self.vs, self.R, self.k, self.vocab
        L = self.logits[:R]
        w = self.win_out
        nws = int(self.ws.numel())
        return (L.data_ptr(), L.stride(0), R, V, self.ctx.data_ptr(), int(self.ctx.numel()),
                self.drafts.data_ptr(), PEN["window"], PEN["repeat"], PEN["presence"], PEN["frequency"],
                self.q_ids.data_ptr(), self.q_raw.data_ptr(), 8, 8, w["q_pen"].data_ptr(),
                CFG["temperature"], CFG["top_k"], CFG["top_p"], CFG["min_p"], self.u.data_ptr(),
                w["pool_vals"].data_ptr(), w["pool_ids"].data_ptr(), *(t.data_ptr() for t in w["p"]),
                *(t.data_ptr() for t in w["q"]), w["tokens"].data_ptr(), w["n"].data_ptr(),
                self.ws.data_ptr() if nws else None, nws)

    def acceptance(self):
        """The acceptance stage as the library runs it: verify_window (two launches)."""
        st = self.vs.library().verify_window(*self._win_args, self.torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"verify_window failed with status {st}")

    def acceptance_separate(self):
        """The same stage as seven separate calls (penalties, top-K, two policies, acceptance)."""
        st = self.torch.cuda.current_stream().cuda_stream
        for fn, a in self._acc_calls:
            if fn is None:
                self.q_vals.copy_(self.q_raw)
                continue
            status = fn(*a, st)
            if status != 0:
                raise RuntimeError(f"acceptance stage call failed with status {status}")

    def step(self):
        self.projections(self.R)
        self.acceptance()


ACCEPT_REPS = 200
GRAPH_SWEEP_R = (1, 4, 8, 9, 16, 17, 24)


def time_region(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps  # ms per call


def time_each(torch, fn, reps, warmup):
    """Per-call times in ms (HIP events around each call on the current stream)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in ev]


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=10):
    """Device-to-device copy of nbytes (torch copy_): GB/s counting bytes read plus written."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ms = float(np.median(time_each(torch, lambda: dst.copy_(src), reps, 2)))
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "ms": round(ms, 4), "gbs_read_plus_write": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def sampling_batch(torch, vs, synth, dev, B=16384, k=3, vocab=4096, steps=10, warmup=2):
    """Batched acceptance stage, one set of rows per window (config: vocab 4096, k = 3)."""
    R = k + 1
    g = torch.Generator(device=dev)
    g.manual_seed(7000)
    p_log = torch.randn((B * R, vocab), generator=g, device=dev) * 3.0
    q_log = 0.9 * p_log.view(B, R, vocab)[:, :k].reshape(B * k, vocab) + \
        (1 - 0.81) ** 0.5 * 3.0 * torch.randn((B * k, vocab), generator=g, device=dev)
    u = torch.rand((B, R, 2), generator=g, device=dev)
    ud = torch.rand((B * k,), generator=g, device=dev)
    pv = torch.empty((B * R, 64), device=dev)
    pi = torch.empty((B * R, 64), dtype=torch.int32, device=dev)
    qv = torch.empty((B * k, 64), device=dev)
    qi = torch.empty((B * k, 64), dtype=torch.int32, device=dev)
    ws_p = torch.empty(max(1, vs.topk_rows_workspace_bytes(B * R, vocab, 64)), dtype=torch.uint8, device=dev)
    ws_q = torch.empty(max(1, vs.topk_rows_workspace_bytes(B * k, vocab, 64)), dtype=torch.uint8, device=dev)
    p_out = (torch.empty((B * R, 64), dtype=torch.int32, device=dev),
             torch.empty((B * R, 64), dtype=torch.float32, device=dev),
             torch.empty((B * R,), dtype=torch.int32, device=dev), None)
    q_out = (torch.empty((B * k, 64), dtype=torch.int32, device=dev),
             torch.empty((B * k, 64), dtype=torch.float32, device=dev),
             torch.empty((B * k,), dtype=torch.int32, device=dev),
             torch.empty((B * k,), dtype=torch.int32, device=dev))
    acc = (torch.empty((B, R), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev))
    acc_f = (torch.empty((B, R), dtype=torch.int32, device=dev), torch.empty((B,), dtype=torch.int32, device=dev))

    def separate():
        vs.topk_rows(p_log, 64, pv, pi, ws_p)
        vs.sample_policy_rows(pv, pi, out=p_out, **CFG)
        vs.topk_rows(q_log, 64, qv, qi, ws_q)
        vs.sample_policy_rows(qv, qi, u=ud, out=q_out, **CFG)
        drafts = q_out[3].view(B, k)
        vs.spec_accept_rows(vs.ACCEPT_SAMPLED, drafts, p_out[:3], q_out[:3], u=u, out=acc)

    def fused():
        vs.verify_windows(p_log, q_log, k, u_draft=ud, u=u, out=acc_f, **CFG)

    # the one-launch stage gives the five calls' bits
    separate()
    fused()
    torch.cuda.synchronize()
    if not (torch.equal(acc[0], acc_f[0]) and torch.equal(acc[1], acc_f[1])):
        raise RuntimeError("verify_windows differs from the separate calls")
    # the two forms in alternating rounds (medians), after a long warm-up: in
    # a fresh process the first timed steps run several percent slow
    for _ in range(10):
        fused()
        separate()
    rounds = [(time_region(torch, fused, steps, warmup), time_region(torch, separate, steps, warmup))
              for _ in range(5)]
    ms = float(np.median([r[0] for r in rounds]))
    ms_sep = float(np.median([r[1] for r in rounds]))
    mean_emitted = float(acc_f[1].float().mean().item())
    nbytes = (B * R + B * k) * vocab * 4  # every target and draft row read once
    return {"windows": B, "k": k, "vocab": vocab, "ms": ms,
            "rows_per_s": B * R / (ms * 1e-3), "windows_per_s": B / (ms * 1e-3),
            "logit_bytes": nbytes, "gb_per_s": nbytes / (ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "kernel": "verify_windows (one launch)",
            "ms_separate_calls": ms_sep, "rows_per_s_separate_calls": B * R / (ms_sep * 1e-3),
            "mean_emitted_per_window": mean_emitted}


def draft_side(torch, vs, synth, dev, steps=50, warmup=5):
    """Draft-side work of one window: the top-16 of 15 draft rows over the
    151936-token vocabulary (with planted near-ties), then greedy acceptance
    of a 15-draft chain and of a 3-branch x depth-8 tree.  Launches go
    straight to the C ABI with cached arguments, so the times are the GPU's."""
    lib = vs.library()
    stream = torch.cuda.current_stream().cuda_stream
    V = synth.VOCAB
    x = torch.from_numpy(synth.topk_planted_rows(8300, rows=15, vocab=V, K=16)).to(dev)
    vals = torch.empty((15, 16), device=dev)
    idx = torch.empty((15, 16), dtype=torch.int32, device=dev)
    nws = vs.topk_rows_workspace_bytes(15, V, 16)
    ws = torch.empty(max(16, nws), dtype=torch.uint8, device=dev)

    def topk():
        st = lib.topk_rows(x.data_ptr(), V, 15, V, 16, vals.data_ptr(), idx.data_ptr(), 16, ws.data_ptr(), nws, stream)
        assert st == 0, st

    ms_topk = time_region(torch, topk, steps, warmup)
    topk_bytes = 15 * V * 4 + 15 * 16 * 8

    def accept_launcher(mode, tokens, p_ids, parent, k):
        tok = torch.empty((1, k + 1), dtype=torch.int32, device=dev)
        n = torch.empty((1,), dtype=torch.int32, device=dev)
        args = (mode, 1, k, p_ids.data_ptr(), None, None, p_ids.shape[1], k + 1, None, None, None, 1, 0,
                tokens.data_ptr(), parent.data_ptr() if parent is not None else None, None,
                tok.data_ptr(), n.data_ptr(), stream)

        def run():
            st = lib.spec_accept_rows(*args)
            assert st == 0, st
        return run

    argmax, drafts = synth.chain_greedy_case(8301, 15, 7)
    p_chain = torch.full((16, 2), -1, dtype=torch.int32, device=dev)
    p_chain[:, 0] = torch.from_numpy(argmax).to(dev)
    d_chain = torch.from_numpy(drafts[None, :]).to(dev)
    ms_chain = time_region(torch, accept_launcher(vs.ACCEPT_GREEDY, d_chain, p_chain, None, 15), steps, warmup)
    parent, tokens, t_am = synth.tree_greedy_case(8302, 3, 8, 1, 5)
    p_tree = torch.full((25, 2), -1, dtype=torch.int32, device=dev)
    p_tree[:, 0] = torch.from_numpy(t_am).to(dev)
    d_tree = torch.from_numpy(tokens[None, :]).to(dev)
    par = torch.from_numpy(parent[None, :]).to(dev)
    ms_tree = time_region(torch, accept_launcher(vs.ACCEPT_GREEDY_TREE, d_tree, p_tree, par, 24), steps, warmup)
    return {"workload": "15 draft rows x 151936, top-16; greedy chain of 15 drafts; greedy tree 3 x 8",
            "topk_us": round(ms_topk * 1e3, 2), "topk_gbs": round(topk_bytes / (ms_topk * 1e-3) / 1e9, 1),
            "greedy_chain_accept_us": round(ms_chain * 1e3, 2),
            "greedy_tree_accept_us": round(ms_tree * 1e3, 2)}


def depth_report(vs, sweep):
    """The draft-depth choice on the measured window cost.

    The cost of a window of r rows is the measured verify pass at R = r
    (projections of the stack and the LM head; no attention).  Reports the
    straight-line fits (base + per_row * (R - 1), least squares over
    R = 1..8 and 1..24), the break-even tokens cost(R) / cost(1), and the
    library's depth choice for constant per-depth acceptance rates.
    """
    Rs = sorted(sweep)
    if len(Rs) < 2 or Rs != list(range(1, len(Rs) + 1)):
        return None
    cost = [float(sweep[r]) for r in Rs]
    x = np.arange(len(Rs), dtype=np.float64)
    fits = {}
    for hi in (8, len(Rs)):
        per_row, base = np.polyfit(x[:hi], np.array(cost[:hi]), 1)
        fits[f"fit_ms_1_{hi}"] = {"base": round(float(base), 4), "per_row": round(float(per_row), 4)}
    kmax = len(Rs) - 1
    return {
        "cost": f"measured verify-pass ms at R = 1..{len(Rs)} (projections only)",
        **fits,
        "break_even_tokens": {str(r): round(cost[r - 1] / cost[0], 4) for r in Rs[1:]},
        "k_star_constant_alpha": {f"{a:.2f}": vs.choose_depth([a] * kmax, cost)[0]
                                  for a in (0.3, 0.5, 0.6, 0.7, 0.8, 0.9, 0.95)},
    }


def lookup_report(vs, synth, length=32768, calls=200):
    """Host latency of drafting a prompt-lookup token tree (3 matches of the
    last 3 tokens, depth 8, 24 nodes) from a context of copied lines."""
    ctx = synth.lookup_context(8200, length + calls)
    sizes = []
    t0 = time.perf_counter()
    for i in range(calls):
        tk, _ = vs.lookup_tree(ctx[:length + i], 3, 3, 8, 24)
        sizes.append(len(tk))
    us = (time.perf_counter() - t0) / calls * 1e6
    return {"context_tokens": length, "us_per_tree": round(us, 1),
            "mean_nodes": round(float(np.mean(sizes)), 2), "host": "one core"}


def host_cpu():
    """(logical CPUs, model name) of this host."""
    model = None
    try:
        import subprocess

        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except Exception:  # pragma: no cover
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:  # pragma: no cover
            pass
    return os.cpu_count(), model


def oracle_gemv_leg(synth, R, budget_s, threads):
    """GB/s of the fp64 projection oracle over one fused layer, repeated for budget_s."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    shapes = list(synth.LAYER_SHAPES_FUSED.values())
    mats = [synth.gemv_case(8000 + i, N, K, R) for i, (N, K) in enumerate(shapes)]
    with threadpool_limits(limits=threads):
        used = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
        done_bytes, spent, calls = 0, 0.0, 0
        while spent < budget_s:
            for (N, K), (w, x) in zip(shapes, mats):
                t0 = time.perf_counter()
                oracle.gemv.gemv_rows(w, x)
                spent += time.perf_counter() - t0
                done_bytes += 2 * N * K + 4 * R * (K + N)
                calls += 1
    return {"gbs": done_bytes / spent / 1e9, "threads": int(used), "calls": calls,
            "gb": done_bytes / 1e9, "seconds": spent}


def cpu_baseline(synth, R, budget_s=8.0):
    """The oracle (as it stands) on a bounded sample of the same pass, on the
    host cores: the projection oracle with every core and with one thread,
    and the acceptance-stage oracle on one window."""
    import oracle

    ncpu, model = host_cpu()
    allc = oracle_gemv_leg(synth, R, budget_s, ncpu)
    one = oracle_gemv_leg(synth, R, budget_s, 1)
    V = synth.VOCAB
    lg = synth.logits(8100, (R, V))
    hot = np.unique(np.argsort(-lg, axis=1)[:, :64])
    ctx = synth.penalty_history(8101, V, 2048, 32, hot)
    q_ids, q_vals = synth.draft_candidates(8102, lg[:R - 1], 8)
    drafts = q_ids[:, 0].copy()
    u = synth.uniforms(8103, (R, 2))
    t0 = time.perf_counter()
    oracle.pipeline.acceptance_stage(lg, ctx, drafts, u, q_ids=q_ids, q_vals=q_vals, **PEN, **CFG)
    acc_s = time.perf_counter() - t0
    batched = oracle_batched_leg(synth)
    return {"value": allc["gbs"], "unit": "GB/s", "cores": allc["threads"], "kind": "oracle",
            "sample": f"fp64 projection oracle on one fused 8B-class layer (qkv, o, gate|up, "
                      f"down), repeated for ~{budget_s:.0f} s per leg ({allc['calls']} calls, "
                      f"{allc['gb']:.2f} GB of bf16 weights with every core; {one['calls']} calls, "
                      f"{one['gb']:.2f} GB on one thread; R={R}); acceptance-stage oracle on one "
                      f"window (R={R}, vocab {V}, single-threaded Python): {acc_s * 1e3:.0f} ms",
            "host_logical_cpus": ncpu,
            "host_cpu_model": model,
            "single_thread": {"value": one["gbs"], "unit": "GB/s", "threads": one["threads"]},
            "seconds": allc["seconds"] + one["seconds"] + acc_s,
            "accept_window_ms": acc_s * 1e3,
            "accept_rows_per_s": R / acc_s,
            "batched_sampling": batched}


def oracle_batched_leg(synth, k=3, vocab=4096, budget_s=4.0):
    """The oracle on windows of the batched sampling workload (k + 1 target
    and k draft rows of `vocab` logits each: top-64 pool, policy, the
    drafts' draws, sampled acceptance), single-threaded, for ~budget_s."""
    import oracle

    R = k + 1
    windows, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        p = synth.logits(8200 + windows, (R, vocab))
        q = synth.logits(8300 + windows, (k, vocab))
        u = synth.uniforms(8400 + windows, (R, 2))
        ud = synth.uniforms(8500 + windows, (k,))
        pv, pi = oracle.topk.topk_rows(p, 64)
        qv, qi = oracle.topk.topk_rows(q, 64)
        p_rows = [oracle.policy.policy_row(pv[i], pi[i], **CFG) for i in range(R)]
        q_rows = [oracle.policy.policy_row(qv[i], qi[i], **CFG) for i in range(k)]
        drafts = [int(q_rows[i][0][oracle.policy.draw(q_rows[i][1], ud[i])]) for i in range(k)]
        oracle.accept.accept_sampled(p_rows, q_rows, drafts, u)
        windows += 1
    secs = time.perf_counter() - t0
    return {"windows": windows, "seconds": secs, "rows_per_s": windows * R / secs,
            "windows_per_s": windows / secs, "threads": 1,
            "sample": f"{windows} windows of k = {k} over {vocab} tokens (the GPU leg's `sampling` workload), "
                      f"single-threaded Python"}


def tree_window_leg(torch, vs, synth, dev):
    """The acceptance stage of one token tree on LM-head rows: a 3 x 8 tree
    (25 rows of 151936 logits, branch tokens planted so that walks go deep),
    per-branch penalties over a 2048 + 32 token history (window 64), the
    top-64 pool, the policy, and the naive-sampling tree walk, through
    verify_tree_window (two launches) and as the four separate calls, both
    with cached C-ABI arguments; the two give the same bits (checked here
    once).  Times are the mean of back-to-back calls (HIP events).  The
    penalties work in place, so later calls see rows already penalised; the
    work per call is the same."""
    V = synth.LM_HEAD_SHAPE[0]
    lg, ctx, tokens, parent, u = synth.tree_window(8200, V)
    R, n = lg.shape[0], len(tokens)
    src = torch.from_numpy(lg).to(dev)
    C, T, P = (torch.from_numpy(a).to(dev) for a in (ctx, tokens, parent))
    U = torch.from_numpy(u[None]).to(dev)
    lib = vs.library()
    pen = (PEN["window"], PEN["repeat"], PEN["presence"], PEN["frequency"])
    cfg = (CFG["temperature"], CFG["top_k"], CFG["top_p"], CFG["min_p"])

    def buffers():
        return dict(L=src.clone(), pv=torch.empty((R, 64), device=dev),
                    pi=torch.empty((R, 64), dtype=torch.int32, device=dev),
                    di=torch.empty((R, 64), dtype=torch.int32, device=dev), dp=torch.empty((R, 64), device=dev),
                    dl=torch.empty((R,), dtype=torch.int32, device=dev),
                    tok=torch.full((1, n + 1), -1, dtype=torch.int32, device=dev),
                    cnt=torch.empty((1,), dtype=torch.int32, device=dev))

    nws = max(vs.topk_rows_workspace_bytes(R, V, 64), vs.verify_window_workspace_bytes(R, V))
    ws = torch.empty(max(16, nws), dtype=torch.uint8, device=dev)
    b1, b2 = buffers(), buffers()
    sep_calls = [
        (lib.penalize_tree_rows, (b1["L"].data_ptr(), None, V, V, V, C.data_ptr(), int(C.numel()), T.data_ptr(),
                                  P.data_ptr(), n, *pen)),
        (lib.topk_rows, (b1["L"].data_ptr(), V, R, V, 64, b1["pv"].data_ptr(), b1["pi"].data_ptr(), 64,
                         ws.data_ptr(), nws)),
        (lib.sample_policy_rows, (b1["pv"].data_ptr(), b1["pi"].data_ptr(), 64, R, 64, *cfg, b1["di"].data_ptr(),
                                  b1["dp"].data_ptr(), b1["dl"].data_ptr(), 64, None, None)),
        (lib.spec_accept_rows, (vs.ACCEPT_NAIVE_TREE, 1, n, b1["di"].data_ptr(), b1["dp"].data_ptr(),
                                b1["dl"].data_ptr(), 64, R, None, None, None, 1, 0, T.data_ptr(), P.data_ptr(),
                                U.data_ptr(), b1["tok"].data_ptr(), b1["cnt"].data_ptr())),
    ]
    fused_args = (b2["L"].data_ptr(), V, R, V, C.data_ptr(), int(C.numel()), T.data_ptr(), P.data_ptr(), *pen,
                  *cfg, U.data_ptr(), b2["pv"].data_ptr(), b2["pi"].data_ptr(), b2["di"].data_ptr(),
                  b2["dp"].data_ptr(), b2["dl"].data_ptr(), b2["tok"].data_ptr(), b2["cnt"].data_ptr(),
                  ws.data_ptr(), nws)

    def separate():
        st = torch.cuda.current_stream().cuda_stream
        for fn, a in sep_calls:
            status = fn(*a, st)
            if status != 0:
                raise RuntimeError(f"tree acceptance call failed with status {status}")

    def fused():
        status = lib.verify_tree_window(*fused_args, torch.cuda.current_stream().cuda_stream)
        if status != 0:
            raise RuntimeError(f"verify_tree_window failed with status {status}")

    separate()
    fused()
    torch.cuda.synchronize()
    for key in ("L", "pv", "pi", "di", "dp", "dl", "tok", "cnt"):
        if not torch.equal(b1[key].view(torch.int32), b2[key].view(torch.int32)):
            raise RuntimeError(f"verify_tree_window differs from the separate calls in {key}")
    emitted = int(b2["cnt"].item())
    us = time_region(torch, fused, ACCEPT_REPS, 5) * 1e3
    us_sep = time_region(torch, separate, ACCEPT_REPS, 5) * 1e3
    return {"config": f"3 x 8 tree ({R} rows of {V}), window {PEN['window']}, top-64 pool, "
                      f"T{CFG['temperature']}/top-k{CFG['top_k']}/top-p{CFG['top_p']}/min-p{CFG['min_p']}, "
                      "naive-sampling walk",
            "us": round(us, 2), "us_separate_calls": round(us_sep, 2),
            "us_note": f"verify_tree_window (two launches) and the four separate calls, each the mean of "
                       f"{ACCEPT_REPS} back-to-back stages (HIP events); same bits, checked at setup",
            "emitted_first_call": emitted}


def tree_attention_leg(torch, vs, synth, dev, reps=20, warmup=3):
    """Attention of a 3-branch x 8-deep token tree (25 rows) under the tree
    mask: 32 query heads over 8 KV heads of 128, a 2080-position context
    (prompt 2048 + 32 emitted) in a 4096-position cache, keys and values
    N(0, 1) bf16, queries N(0, 1) fp32.  C-ABI calls with cached arguments:
    the mean of back-to-back calls and the median of `reps` single calls.
    Algorithmic bytes: the context's keys and values once, the scratch
    slots, queries and outputs once."""
    R, Hq, Hkv, D, ctx, L = 25, 32, 8, 128, 2080, 4096
    g = torch.Generator(device=dev)
    g.manual_seed(7100)
    q = torch.randn((R, Hq, D), generator=g, device=dev, dtype=torch.float32)
    kc = torch.randn((Hkv, L, D), generator=g, device=dev).to(torch.bfloat16)
    vc = torch.randn((Hkv, L, D), generator=g, device=dev).to(torch.bfloat16)
    ks = torch.randn((Hkv, R, D), generator=g, device=dev).to(torch.bfloat16)
    vs_ = torch.randn((Hkv, R, D), generator=g, device=dev).to(torch.bfloat16)
    parent = torch.tensor([-1 if j % 8 == 0 else j - 1 for j in range(R - 1)], dtype=torch.int32, device=dev)
    out = torch.empty((R, Hq, D), dtype=torch.float32, device=dev)
    nws = vs.tree_attention_rows_workspace_bytes(R, Hq, Hkv, ctx)
    ws = torch.empty(max(16, nws), dtype=torch.uint8, device=dev)
    scale = 1.0 / float(np.sqrt(D))
    vs.tree_attention_rows(q, kc, vc, ctx, ks, vs_, parent, scale=scale, out=out, workspace=ws)  # checks the arguments
    lib = vs.library()
    args = (q.data_ptr(), R, Hq, D, kc.data_ptr(), vc.data_ptr(), L, ctx, ks.data_ptr(), vs_.data_ptr(), R,
            parent.data_ptr(), Hkv, scale, out.data_ptr(), ws.data_ptr(), int(ws.numel()))

    def call():
        st = lib.tree_attention_rows(*args, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"tree_attention_rows failed with status {st}")

    us_single = float(np.median(time_each(torch, call, reps, warmup))) * 1e3
    us = time_region(torch, call, ACCEPT_REPS, warmup) * 1e3  # back to back, as a pipeline enqueues it
    nbytes = 2 * Hkv * ctx * D * 2 + 2 * Hkv * R * D * 2 + 2 * R * Hq * D * 4
    return {"config": f"3 x 8 tree ({R} rows), {Hq}/{Hkv} heads of {D}, context {ctx}",
            "us": round(us, 2), "us_note": f"mean of {ACCEPT_REPS} back-to-back calls (HIP events); "
                                           "us_single_call: median of single calls, each bracketed by events",
            "us_single_call": round(us_single, 2), "algorithmic_bytes": nbytes,
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "hbm_floor_us": round(nbytes / (HBM_PEAK_GBS * 1e9) * 1e6, 2)}


def family_sweep(torch, vs, synth, dev, reps=12, warmup=3):
    """verify_gemv_rows alone on every fused projection and LM head of three
    model sizes, each R = 1..24: median of `reps` HIP-event-timed calls after
    `warmup`, with the matrix's algorithmic bytes over that time as a
    fraction of the 8 TB/s peak.  Weights N(0, 0.02) bf16, activations
    N(0, 1); the workspace is passed where the dispatch uses one."""
    lib = vs.library()
    X = torch.randn(24, max(K for f in synth.FAMILY_SHAPES.values() for _, K in f.values()),
                    device=dev, dtype=torch.float32)
    out = {}
    for fam, shapes in synth.FAMILY_SHAPES.items():
        for name, (N, K) in shapes.items():
            W = (torch.randn(N, K, device=dev) * 0.02).to(torch.bfloat16)
            Y = torch.empty(24, N, device=dev, dtype=torch.float32)
            nws = max(vs.verify_gemv_rows_workspace_bytes(N, K, R) for R in range(1, 25))
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
            per = {}
            for R in range(1, 25):
                need = vs.verify_gemv_rows_workspace_bytes(N, K, R)
                args = (W.data_ptr(), K, N, K, X.data_ptr(), X.stride(0), R, Y.data_ptr(), N,
                        ws.data_ptr() if need else None, need)

                def call():
                    st = lib.verify_gemv_rows(*args, torch.cuda.current_stream().cuda_stream)
                    if st != 0:
                        raise RuntimeError(f"verify_gemv_rows failed with status {st}")

                us = float(np.median(time_each(torch, call, reps, warmup))) * 1e3
                nbytes = 2 * N * K + 4 * R * (K + N)
                per[str(R)] = {"us": round(us, 2), "frac_of_hbm_peak": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 3),
                               "kernel": "split-K" if need else "row-block"}
            out[f"{fam}/{name}"] = {"N": N, "K": K, "vs_R": per}
            log(f"{fam}/{name} {N}x{K}: R1 {per['1']['frac_of_hbm_peak']}, R4 {per['4']['frac_of_hbm_peak']}, "
                f"R24 {per['24']['frac_of_hbm_peak']}")
            del W, Y, ws
            torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the verify step would shard the projections by output rows and the "
              "top-K by vocabulary slices)", file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    import verify_sampling_amd as vs

    vs.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.family_sweep:
        fam = family_sweep(torch, vs, synth, dev)
        print(json.dumps({"metric": "verify_gemv_rows fraction of HBM peak per matrix, three model sizes",
                          "unit": "fraction of 8 TB/s", "data": "synthetic", "n_gpus": 1,
                          "timing": "median of 12 HIP-event-timed calls after 3 warm-ups per R",
                          "family_sweep": fam}), flush=True)
        return
    if args.copy_calibration:
        src = torch.ones(CALIB_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    R = args.rows
    rmax = 24
    log(f"generating weights: {args.layers} layers + LM head")
    t0 = time.time()
    vp = VerifyPass(torch, vs, synth, args.layers, rmax, dev)
    log(f"weights ready in {time.time() - t0:.1f}s")
    vp.setup_acceptance(synth, R)

    def captured(fn):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for _ in range(2):
                fn()
        torch.cuda.current_stream().wait_stream(s)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        return graph

    def captured_step():
        return captured(vp.step)

    graph = captured_step() if args.graph else None
    step = graph.replay if args.graph else vp.step
    ms_step = time_region(torch, step, args.steps, max(args.warmup, 30) if args.graph else args.warmup)
    step_bytes = vp.bytes_projections(R)
    log(f"step: {ms_step:.3f} ms")
    if args.projections_only:
        ms_proj = time_region(torch, lambda: vp.projections(R), args.steps, args.warmup)
        print(json.dumps({"metric": "verify pass (projections only, a profiling run)", "rows": R,
                          "layers": args.layers, "ms_per_step": ms_step, "ms_projections": ms_proj,
                          "projection_gb_per_s": step_bytes / (ms_proj * 1e-3) / 1e9}), flush=True)
        return
    # the other form of the same step: replayed as a HIP graph (or eager, under
    # --graph).  The GPU idles while the host captures, and its clocks need
    # ~30 steps to come back up, hence the longer warm-up.
    if args.graph:
        ms_step_other = time_region(torch, vp.step, args.steps, max(args.warmup, 30))
    else:
        graph = captured_step()
        ms_step_other = time_region(torch, graph.replay, args.steps, max(args.warmup, 30))
    del graph
    log(f"step ({'eager' if args.graph else 'HIP graph'}): {ms_step_other:.3f} ms")

    # the projection kernel alone, for the roofline (same stream, HIP events)
    ms_proj = time_region(torch, lambda: vp.projections(R), args.steps, args.warmup)
    # the acceptance stage is ~20 us: 200 back-to-back calls, so that the host's
    # latency before the first launch is not spread over only a few calls
    ms_accept = time_region(torch, vp.acceptance, ACCEPT_REPS, args.warmup)
    ms_accept_sep = time_region(torch, vp.acceptance_separate, ACCEPT_REPS, args.warmup)
    # the same 200 calls replayed as one HIP graph: the GPU's time per stage
    # without the host's per-call launch work (the eager figure above can be
    # bound by the host issuing 200 calls of 34 arguments each)
    def accept_batch():
        for _ in range(ACCEPT_REPS):
            vp.acceptance()
    g_acc = captured(accept_batch)
    ms_accept_graph = float(np.median(time_each(torch, g_acc.replay, 10, 30))) / ACCEPT_REPS
    del g_acc
    per_launch_ms = ms_proj / vp.n_launches()
    bytes_per_launch = step_bytes / vp.n_launches()
    achieved = bytes_per_launch / (per_launch_ms * 1e-3) / 1e9

    sweep, spread, sweep_graph = {}, {}, {}
    if not args.no_sweep:
        for r in range(1, 25):
            ts = time_each(torch, lambda: vp.projections(r), max(10, args.steps // 2), 2)
            sweep[r] = float(np.median(ts))
            spread[r] = (float(np.min(ts)), float(np.max(ts)), len(ts))
        # the same passes replayed as HIP graphs (launches recorded once)
        for r in GRAPH_SWEEP_R:
            g = captured(lambda: vp.projections(r))
            sweep_graph[r] = float(np.median(time_each(torch, g.replay, 10, 30)))
            del g
        log("sweep done")
    knee = None
    if sweep:
        t1 = sweep[1]
        knee = next((r for r in sorted(sweep) if sweep[r] > 1.1 * t1), None)

    copy = copy_bandwidth(torch, dev)
    log(f"device copy: {copy['gbs_read_plus_write']} GB/s (read + write)")
    sampling = None if args.no_sampling else sampling_batch(torch, vs, synth, dev)
    if sampling:
        log(f"sampling: {sampling['rows_per_s']:.3e} rows/s")
    draft = None if args.no_sampling else draft_side(torch, vs, synth, dev)
    tree_attn = tree_attention_leg(torch, vs, synth, dev)
    log(f"tree attention: {tree_attn['us']} us ({tree_attn['frac_of_hbm_peak']} of peak)")
    tree_win = tree_window_leg(torch, vs, synth, dev)
    log(f"tree acceptance stage: {tree_win['us']} us ({tree_win['us_separate_calls']} us as four calls)")

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(synth, R)

    out = {
        "metric": "verify-pass HBM GB/s (ms/pass vs rows R=1..24; accepted-token sampling rows/s)",
        "value": step_bytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16xf32",
        "data": "synthetic",
        "config": {
            "workload": f"verify window: {args.layers}-layer 8B-class projection stack "
                        f"(qkv 6144x4096, o 4096x4096, gate|up 24576x4096, down 4096x12288) "
                        f"+ LM head 151936x4096 + acceptance stage (penalties W=64, top-64 pool, "
                        f"T0.7/top-k20/top-p0.95/min-p0.05, rejection accept), R={R}",
            "rows": R,
            "layers": args.layers,
            "bytes_per_pass": step_bytes,
            "graph": bool(args.graph),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": ("verify_gemv_rows: gemv_rows_staged_kernel (staged row-block)" if R <= 8 else
                       "verify_gemv_rows: gemv_rows_staged_kernel and gemv_shared_kernel (split-K) with reduce_partials_kernel"),
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "frac_of_measured_copy": achieved / copy["gbs_read_plus_write"],
            "traffic": measured_traffic(R),
            "traffic_unit": "HBM bytes per projection call (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "traffic_vs_R": {str(r): measured_traffic(r) for r in (4, 9, 16, 17, 24)},
            "launches_per_pass": vp.n_launches(),
            "avg_launch_us": per_launch_ms * 1e3,
        },
        "ms_projections": ms_proj,
        "ms_per_step_graph" if not args.graph else "ms_per_step_eager": ms_step_other,
        "ms_acceptance": ms_accept,
        "ms_acceptance_note": "verify_window, the whole acceptance stage of the window in two launches "
                              "(bit-identical to the separate calls, checked at setup); "
                              "ms_acceptance_separate_calls: the same stage as seven library calls; "
                              f"both the mean of {ACCEPT_REPS} back-to-back calls (HIP events); "
                              "ms_acceptance_graph: the same calls replayed as one HIP graph (no host launch work)",
        "ms_acceptance_separate_calls": ms_accept_sep,
        "ms_acceptance_graph": ms_accept_graph,
        "verify_rows_per_s": R / (ms_step * 1e-3),
        "emitted_tokens_per_s": (sampling["mean_emitted_per_window"] / (ms_step * 1e-3)
                                 if sampling else None),
        "emitted_tokens_note": "verify windows per second times the mean tokens emitted per window "
                               "of the batched sampling stage (synthetic q with correlation 0.9 "
                               "to p; no trained draft model)",
        "device_copy": copy,
        "sweep_timing": "median of per-pass HIP-event times, "
                        f"{max(10, args.steps // 2)} passes after 2 warm-ups per R",
        "ms_per_pass_vs_R": {str(r): round(v, 4) for r, v in sweep.items()},
        "ms_per_pass_graph_vs_R": {str(r): round(v, 4) for r, v in sweep_graph.items()},
        "ms_per_pass_min_max_vs_R": {str(r): [round(a, 4), round(b, 4)]
                                     for r, (a, b, _) in spread.items()},
        "gbs_vs_R": {str(r): round(vp.bytes_projections(r) / (v * 1e-3) / 1e9, 1)
                     for r, v in sweep.items()},
        "frac_of_hbm_peak_vs_R": {str(r): round(vp.bytes_projections(r) / (v * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)
                                  for r, v in sweep.items()},
        "frac_of_measured_copy_vs_R": {
            str(r): round(vp.bytes_projections(r) / (v * 1e-3) / 1e9 / copy["gbs_read_plus_write"], 4)
            for r, v in sweep.items()},
        "verify_rows_per_s_vs_R": {str(r): round(r / (v * 1e-3), 1) for r, v in sweep.items()},
        "knee_R": knee,
        "depth_chooser": depth_report(vs, sweep) if sweep else None,
        "prompt_lookup_drafter": lookup_report(vs, synth),
        "sampling": sampling,
        "draft_side": draft,
        "tree_attention": tree_attn,
        "tree_window": tree_win,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
