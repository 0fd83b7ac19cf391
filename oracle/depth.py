"""The draft-depth chooser and the window-cost model.

[SD] "Speculative decoding on RDNA", §05 "What a verify row costs on RDNA":
a window of R verify rows (k = R - 1 drafts plus the current position) costs
a measured amount; dividing it by the one-row cost (a plain decode step)
gives the tokens the window must emit to break even with plain decoding.
The page's fits are linear in the rows: cost(R) = base + per_row * (R - 1).
The depth is chosen per window as the k that maximises the expected emitted
tokens, 1 plus the running products of the per-depth acceptance rates, per
unit of window cost, falling back to one token per step (k = 0) when no
window beats it.

Readings taken:
  * alpha[j - 1] is the probability that draft j is accepted given drafts
    1..j-1 were; expected emitted tokens E(k) = 1 + sum_{j=1..k}
    prod_{i=1..j} alpha[i - 1] (the accepted drafts plus the one token every
    window emits);
  * cost[r - 1] is the cost of a window of r rows; the rate of depth k is
    E(k) / cost[k];
  * ties go to the smaller k (fewer rows for the same rate);
  * all arithmetic in fp64, the running product and sum in increasing j.

Test infrastructure only: imported by tests/ and bench.py's reporting, never
by the library.
"""

from __future__ import annotations


def linear_window_cost(base: float, per_row: float, rows: int) -> float:
    """cost(R) = base + per_row * (R - 1) (the page's fitted form)."""
    return float(base) + float(per_row) * (rows - 1)


def break_even_tokens(cost, rows: int) -> float:
    """Tokens a window of `rows` rows must emit to match plain decoding: cost(R) / cost(1)."""
    return float(cost[rows - 1]) / float(cost[0])


def expected_emitted(alpha, k: int) -> float:
    """1 + sum_{j=1..k} prod_{i=1..j} alpha[i-1], accumulated in increasing j."""
    total = 1.0
    run = 1.0
    for j in range(k):
        run = run * float(alpha[j])
        total = total + run
    return total


def choose_depth(alpha, cost, kmax: int):
    """(k*, rate): the depth 0 <= k <= kmax with the largest E(k) / cost[k]."""
    best_k, best_rate = 0, expected_emitted(alpha, 0) / float(cost[0])
    for k in range(1, kmax + 1):
        rate = expected_emitted(alpha, k) / float(cost[k])
        if rate > best_rate:
            best_k, best_rate = k, rate
    return best_k, best_rate
