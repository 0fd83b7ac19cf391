"""Seeded generators for every workload of the verify step.

Every generator takes an integer seed and draws from numpy's PCG64, so a
case is reproduced from its seed alone.  Nothing here computes any part of
the verify step: the bf16 encoding below is how the synthetic weights are
stored, and the planted history tokens and draft candidates are
constructions of input structure (which tokens repeat, which tokens a
drafter would propose), not penalties, pools or distributions.

Recipes (the workloads' shapes and value distributions):
  * weights: N(0, 0.02) fp32, rounded to bf16 (round to nearest even);
  * activations: N(0, 1) fp32, one row per verify row;
  * target logits: N(0, 3) fp32 over the vocabulary;
  * draft logits for the distribution tests: q = rho*p + sqrt(1-rho^2)*eps,
    eps ~ N(0, 3), which keeps q's N(0, 3) marginal while making p and q
    overlap (independent rows over 4096 tokens with top-20 pools almost
    never share support, and then the residual equals p);
  * uniform draws: float32 multiples of 2^-24 in [0, 1) (numpy's float32
    uniform takes the top 24 bits of a 32-bit draw), exact in fp32 and fp64;
  * draft-side top-K rows: N(0, 4) with planted exact ties, 1-ulp
    neighbours, duplicated maxima, -inf, NaN, +-0, an all-equal row and a
    row with fewer finite values than K;
  * prompt-lookup contexts: a coding agent's context is full of
    near-identical lines, so the token stream is a sequence of "lines"
    (6-20 tokens) drawn with Zipf-like popularity from a pool in which
    families of lines share a prefix and differ after it.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "rng",
    "f32_to_bf16_bits",
    "gemv_case",
    "uniforms",
    "logits",
    "correlated_logits",
    "penalty_history",
    "draft_candidates",
    "topk_planted_rows",
    "chain_greedy_case",
    "tree_greedy_case",
    "tree_window",
    "torch_bf16_weights",
    "lookup_context",
    "LAYER_SHAPES",
    "LAYER_SHAPES_FUSED",
    "LM_HEAD_SHAPE",
    "FAMILY_SHAPES",
    "N_LAYERS",
    "VOCAB",
]

# One 8B-class decoder layer in nn.Linear layout W[N][K] (out, in).
LAYER_SHAPES = {
    "q": (4096, 4096),
    "k": (1024, 4096),
    "v": (1024, 4096),
    "o": (4096, 4096),
    "gate": (12288, 4096),
    "up": (12288, 4096),
    "down": (4096, 12288),
}
# The same layer with the projections that read the same activation stored
# as one matrix: q|k|v share the normed hidden state, gate|up share the
# post-attention normed state.
LAYER_SHAPES_FUSED = {
    "qkv": (6144, 4096),
    "o": (4096, 4096),
    "gate_up": (24576, 4096),
    "down": (4096, 12288),
}
N_LAYERS = 36
VOCAB = 151936
LM_HEAD_SHAPE = (VOCAB, 4096)

# The fused projections and the LM head of two other sizes of the same model
# family (hidden 2560 with MLP width 9728, hidden 5120 with 17408; 32 and 40
# query heads of 128, 8 KV heads), for the dispatch's parity and timing
# beyond the 8B-class shapes.
FAMILY_SHAPES = {
    "hidden2560": {"qkv": (6144, 2560), "o": (2560, 4096), "gate_up": (19456, 2560),
                   "down": (2560, 9728), "lm_head": (VOCAB, 2560)},
    "hidden4096": {**LAYER_SHAPES_FUSED, "lm_head": LM_HEAD_SHAPE},
    "hidden5120": {"qkv": (7168, 5120), "o": (5120, 5120), "gate_up": (34816, 5120),
                   "down": (5120, 17408), "lm_head": (VOCAB, 5120)},
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.

    NaN inputs are not produced by the generators and are not handled.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def gemv_case(seed: int, N: int, K: int, R: int, w_std: float = 0.02):
    """W bits [N][K] (bf16 as uint16) ~ N(0, w_std), X [R][K] fp32 ~ N(0, 1)."""
    g = rng(seed)
    w = g.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)
    x = g.standard_normal((R, K), dtype=np.float32)
    return f32_to_bf16_bits(w), x


def uniforms(seed: int, shape) -> np.ndarray:
    """float32 uniforms in [0, 1), each a multiple of 2^-24."""
    return rng(seed).random(shape, dtype=np.float32)


def logits(seed: int, shape, std: float = 3.0) -> np.ndarray:
    return (rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def correlated_logits(p_logits: np.ndarray, rho: float, seed: int, std: float = 3.0) -> np.ndarray:
    """q = rho*p + sqrt(1 - rho^2)*eps, eps ~ N(0, std^2), in fp32."""
    eps = logits(seed, p_logits.shape, std)
    a = np.float32(rho)
    b = np.float32(np.sqrt(max(0.0, 1.0 - rho * rho)))
    return (a * p_logits.astype(np.float32) + b * eps).astype(np.float32)


def penalty_history(seed: int, vocab: int, prompt_len: int, emitted_len: int,
                    hot_tokens: np.ndarray, hot_frac: float = 0.25) -> np.ndarray:
    """prompt || emitted token ids (int32).

    A fraction ``hot_frac`` of the positions is drawn (with repeats) from
    ``hot_tokens`` (for example the highest-logit ids of the target rows),
    so that the window actually touches the tokens a sampler would pick;
    the rest are uniform over the vocabulary.
    """
    g = rng(seed)
    n = prompt_len + emitted_len
    ids = g.integers(0, vocab, size=n, dtype=np.int64)
    hot = g.random(n) < hot_frac
    if len(hot_tokens):
        ids[hot] = g.choice(np.asarray(hot_tokens, dtype=np.int64), size=int(hot.sum()))
    return ids.astype(np.int32)


def tree_window(seed: int, vocab: int = VOCAB, branches: int = 3, depth: int = 8):
    """A token tree's verify rows: branches x depth nodes under the root.

    Node j = depth * b + d (branch b, depth d) hangs under the root (d = 0)
    or node j - 1, and holds the b-th largest raw logit of its parent's row
    (row 0 for the root, row j for node j - 1), raised by a random amount
    that is larger on the lower branches, so that walks go deep.  Also a
    2048 + 32 token history a quarter of which comes from the rows' top 64
    ids, and uniforms [rows][2].  Returns (logits fp32 [n + 1][vocab],
    ctx int32, tokens int32 [n], parent int32 [n], u fp32 [n + 1][2]).
    """
    g = rng(seed)
    n = branches * depth
    lg = logits(seed, (n + 1, vocab))
    tokens = np.zeros(n, dtype=np.int32)
    parent = np.zeros(n, dtype=np.int32)
    for b in range(branches):
        for d in range(depth):
            j = depth * b + d
            parent[j] = -1 if d == 0 else j - 1
            prow = 0 if d == 0 else j
            t = int(np.argsort(-lg[prow], kind="stable")[b])
            tokens[j] = t
            lg[prow, t] += np.float32(2.0 * (branches - b) * g.random())
    hot = np.unique(np.argsort(-lg, axis=1)[:, :64])
    ctx = penalty_history(seed + 1, vocab, 2048, 32, hot)
    u = uniforms(seed + 2, (n + 1, 2))
    return lg, ctx, tokens, parent, u


def draft_candidates(seed: int, target_logits: np.ndarray, n_cand: int = 8, noise_std: float = 0.5):
    """A drafter's re-scored candidate list for each row.

    For row i the candidates are the n_cand largest entries of
    (target row i + N(0, noise_std^2)), and their draft logits are those
    perturbed values.  Returns (ids int32 [rows][n_cand], vals fp32 [rows][n_cand]).
    """
    g = rng(seed)
    rows, vocab = target_logits.shape
    noisy = (target_logits.astype(np.float32)
             + g.standard_normal((rows, vocab), dtype=np.float32) * np.float32(noise_std))
    ids = np.argsort(-noisy, axis=1, kind="stable")[:, :n_cand].astype(np.int32)
    vals = np.take_along_axis(noisy, ids.astype(np.int64), axis=1).astype(np.float32)
    return ids, vals


def topk_planted_rows(seed: int, rows: int = 15, vocab: int = VOCAB, K: int = 16,
                      std: float = 4.0) -> np.ndarray:
    """Draft-side logits [rows][vocab] ~ N(0, std^2) with planted hard cases.

    Per row: exact ties straddling rank K, 1-ulp neighbours of the K-th
    value, a duplicated maximum, a few -inf and NaN entries and +-0.
    Row 1 is all equal; row 2 has fewer than K finite values (the rest
    -inf, with one NaN).
    """
    g = rng(seed)
    x = (g.standard_normal((rows, vocab), dtype=np.float32) * np.float32(std)).astype(np.float32)
    for r in range(rows):
        row = x[r]
        order = np.argsort(-row, kind="stable")
        kth = row[order[K - 1]]
        # exact ties straddling rank K at scattered positions
        pos = g.choice(vocab, size=6, replace=False)
        row[pos] = kth
        # 1-ulp neighbours of the K-th value
        pos = g.choice(vocab, size=4, replace=False)
        row[pos[:2]] = np.nextafter(kth, np.float32(np.inf), dtype=np.float32)
        row[pos[2:]] = np.nextafter(kth, np.float32(-np.inf), dtype=np.float32)
        # duplicated maximum
        mx = row[order[0]]
        row[g.choice(vocab, size=2, replace=False)] = mx
        # specials
        row[g.choice(vocab, size=3, replace=False)] = -np.inf
        row[g.choice(vocab, size=3, replace=False)] = np.nan
        row[g.choice(vocab, size=2, replace=False)] = 0.0
        row[g.choice(vocab, size=2, replace=False)] = -0.0
    if rows > 1:
        x[1, :] = np.float32(1.25)
    if rows > 2:
        x[2, :] = -np.inf
        keep = g.choice(vocab, size=K // 2, replace=False)
        x[2, keep] = g.standard_normal(K // 2, dtype=np.float32)
        x[2, g.integers(0, vocab)] = np.nan
    return x


def chain_greedy_case(seed: int, n_drafts: int, accept_len: int, vocab: int = VOCAB):
    """A greedy chain with a planted accept length.

    Returns (target_argmax int32 [n_drafts+1], drafts int32 [n_drafts]):
    drafts[i] == target_argmax[i] for i < accept_len and differs at
    accept_len (when accept_len < n_drafts).
    """
    g = rng(seed)
    argmax = g.integers(0, vocab, size=n_drafts + 1).astype(np.int32)
    drafts = argmax[:n_drafts].copy()
    if accept_len < n_drafts:
        drafts[accept_len] = (argmax[accept_len] + 1 + g.integers(0, vocab - 1)) % vocab
        tail = g.integers(0, vocab, size=n_drafts - accept_len - 1)
        drafts[accept_len + 1:] = tail
    return argmax, drafts.astype(np.int32)


def tree_greedy_case(seed: int, branches: int, depth: int, match_branch: int, match_len: int,
                     vocab: int = VOCAB):
    """A token tree of `branches` chains of `depth` nodes hanging off the root.

    Node numbering is branch-major: node b*depth + j is branch b at depth j,
    its parent is the root (-1) for j = 0, else node b*depth + j - 1.  Row 0
    of the target is the root, row 1 + node is that node's row.
    ``match_branch`` < 0 plants no match.  Otherwise the target's argmax
    agrees with that branch for its first ``match_len`` nodes, and every
    other branch is made to disagree at its first node.
    Returns (parent int32 [n], tokens int32 [n], target_argmax int32 [n+1]).
    """
    g = rng(seed)
    n = branches * depth
    parent = np.empty(n, dtype=np.int32)
    for b in range(branches):
        for j in range(depth):
            parent[b * depth + j] = -1 if j == 0 else b * depth + j - 1
    tokens = g.integers(0, vocab, size=n).astype(np.int32)
    argmax = g.integers(0, vocab, size=n + 1).astype(np.int32)
    # make all first-level tokens distinct from each other and from the root's argmax
    firsts = g.choice(vocab, size=branches + 1, replace=False).astype(np.int32)
    argmax[0] = firsts[0]
    for b in range(branches):
        tokens[b * depth] = firsts[b + 1]
    if match_branch >= 0 and match_len > 0:
        b = match_branch
        argmax[0] = tokens[b * depth]
        for j in range(1, min(match_len, depth)):
            node_prev = b * depth + j - 1
            argmax[1 + node_prev] = tokens[b * depth + j]
        if match_len < depth:
            last = b * depth + match_len - 1
            nxt = b * depth + match_len
            if argmax[1 + last] == tokens[nxt]:
                argmax[1 + last] = (tokens[nxt] + 1) % vocab
    return parent, tokens, argmax


def torch_bf16_weights(shape, seed: int, device, std: float = 0.02):
    """N(0, std) bf16 weights generated on `device` with a seeded torch.Generator.

    Used for workloads too large to generate on the host (tens of GB).  The
    conversion to bfloat16 rounds to nearest even.
    """
    import torch

    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    w = torch.empty(shape, dtype=torch.float32, device=device)
    w.normal_(0.0, std, generator=gen)
    return w.to(torch.bfloat16)


def lookup_context(seed: int, length: int, vocab: int = VOCAB, families: int = 60,
                   variants: int = 4) -> np.ndarray:
    """int32 token stream of `length` tokens built from repeated near-identical lines.

    Each family has a shared prefix of 3-8 tokens and `variants` different
    tails of 3-12 tokens; lines are drawn with probability proportional to
    1 / (rank + 1) over all family variants.
    """
    g = rng(seed)
    lines = []
    for _ in range(families):
        head = g.integers(0, vocab, size=int(g.integers(3, 9)))
        for _ in range(variants):
            lines.append(np.concatenate([head, g.integers(0, vocab, size=int(g.integers(3, 13)))]))
    w = 1.0 / (np.arange(len(lines)) + 1.0)
    w /= w.sum()
    out = []
    total = 0
    while total < length:
        line = lines[int(g.choice(len(lines), p=w))]
        out.append(line)
        total += len(line)
    return np.concatenate(out)[:length].astype(np.int32)
