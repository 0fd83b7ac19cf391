"""The sampler policy and the inverse-CDF draw.

[SD] "Speculative decoding on RDNA", §03 "how hipfire does it": p is the
AR sampler's distribution: temperature, then the request's top-k (absent
means 20 candidates, 0 means the whole 64-wide pool), then min-p, then
top-p, with the same pool, tie order and summation; q is the same policy
applied to the draft's re-scored candidates and their exact logits; one
request-seeded random stream supplies every draw.

Readings taken where the page is silent:
  * candidate slots with a negative id are empty and ignored; the rest
    are ordered by value descending, then id ascending, NaN
    last (the pool order of oracle.topk); for p the candidates are the
    top-64 of the penalised row;
  * temperature 0 is greedy: all mass on the first candidate;
  * top-k: absent (< 0) -> 20; 0 -> 64; else min(top_k, 64), and never
    more than the candidates given;
  * weights e_j = exp((l_j - l_0) / T) in fp64, l_0 the first (largest)
    logit; -inf and NaN logits get weight 0; if l_0 = +inf, every +inf
    candidate gets weight 1 and the rest 0; if no candidate has a usable
    logit, all mass goes to the first candidate;
  * candidates whose weight is 0 carry no mass and are dropped;
  * min-p keeps j with p_j >= min_p * p_0 (relative to the most likely
    candidate, after temperature);
  * top-p keeps j while the probability mass before j is < top_p, so the
    candidate that crosses top_p is kept and at least one always is;
    top_p >= 1 keeps every candidate;
  * the distribution is renormalised after each filter.  Both filters
    compare ratios of weights, so they are evaluated on the unnormalised
    weights (min-p: e_j >= min_p * e_0; top-p: (sum of kept e before j)
    < top_p * (sum of kept e)) and normalised once at the end;
  * every sum runs sequentially in pool order, in fp64; the output
    probabilities are rounded once to fp32.
The draw returns the first j whose cumulative weight exceeds u times the
total, summed sequentially in fp64 from the given weights.
"""

from __future__ import annotations

import math

import numpy as np

from .topk import order_key

POOL = 64
TOPK_ABSENT = 20


def pool_order(vals: np.ndarray, ids: np.ndarray) -> list[int]:
    """Positions of the candidates in pool order (value desc, id asc, NaN last)."""
    return sorted(range(len(vals)), key=lambda m: order_key(vals[m], int(ids[m])) + (m,))


def effective_top_k(top_k: int) -> int:
    if top_k < 0:
        return TOPK_ABSENT
    if top_k == 0:
        return POOL
    return min(int(top_k), POOL)


def weights(vals: list[float], temperature: float) -> list[float]:
    """e_j for candidates already in pool order (see module doc)."""
    l0 = vals[0]
    T = float(np.float32(temperature))
    if math.isinf(l0) and l0 > 0:
        return [1.0 if (math.isinf(v) and v > 0) else 0.0 for v in vals]
    if not math.isfinite(l0):
        return []
    return [math.exp((v - l0) / T) if math.isfinite(v) else 0.0 for v in vals]


def policy_row(vals, ids, temperature: float, top_k: int, top_p: float, min_p: float):
    """One row's sampling distribution.

    vals: fp32 candidate logits, ids: their token ids (any order, <= 64
    used; negative ids are empty slots and are ignored).
    Returns (ids int32 [L], probs fp32 [L]) in pool order; L >= 1 unless
    every slot is empty.
    """
    vals = np.asarray(vals, dtype=np.float32)
    ids = np.asarray(ids, dtype=np.int32)
    real = ids >= 0  # negative ids mark empty candidate slots
    vals, ids = vals[real], ids[real]
    if len(ids) == 0:
        return np.zeros(0, dtype=np.int32), np.zeros(0, dtype=np.float32)
    order = pool_order(vals, ids)
    v = [float(vals[m]) for m in order]
    t = [int(ids[m]) for m in order]
    if float(np.float32(temperature)) <= 0.0:
        return np.array(t[:1], dtype=np.int32), np.array([1.0], dtype=np.float32)
    n = min(effective_top_k(top_k), len(v))
    v, t = v[:n], t[:n]
    e = weights(v, temperature)
    if not e or e[0] <= 0.0:
        return np.array(t[:1], dtype=np.int32), np.array([1.0], dtype=np.float32)
    # candidates of weight 0 carry no mass and are dropped
    # min-p, relative to the most likely candidate
    mp = float(np.float32(min_p))
    keep = [j for j in range(n) if e[j] > 0.0 and e[j] >= mp * e[0]]
    # top-p on the kept candidates, in pool order; top_p >= 1 keeps all
    tp = float(np.float32(top_p))
    if tp >= 1.0:
        kept2 = keep
    else:
        s = 0.0
        for j in keep:
            s += e[j]
        kept2 = []
        c = 0.0
        for j in keep:
            if c < tp * s or not kept2:
                kept2.append(j)
                c += e[j]
            else:
                break
    z = 0.0
    for j in kept2:
        z += e[j]
    probs = np.array([e[j] / z for j in kept2], dtype=np.float64).astype(np.float32)
    out_ids = np.array([t[j] for j in kept2], dtype=np.int32)
    return out_ids, probs


def draw_weights(w, u: float) -> int:
    """First j with u * total < C_j, C_j the sequential fp64 cumulative sum."""
    c = []
    acc = 0.0
    for x in w:
        acc += float(x)
        c.append(acc)
    target = float(np.float32(u)) * acc
    for j, cj in enumerate(c):
        if target < cj:
            return j
    last = [j for j, x in enumerate(w) if float(x) > 0.0]
    return last[-1] if last else 0


def draw(probs_f32, u: float) -> int:
    """Inverse-CDF draw over a distribution stored in fp32."""
    return draw_weights([float(p) for p in np.asarray(probs_f32, dtype=np.float32)], u)
