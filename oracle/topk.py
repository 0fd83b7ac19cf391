"""Per-row top-K in the pool order.

[SD] "Speculative decoding on RDNA", §03 "how hipfire does it": the sampler
works on a 64-wide candidate pool with a fixed tie order.  [PR] "feat
(dflash): developer-only online draft tuning", "Code map": the batched
top-K over draft rows is gated on byte identity with ties, NaN and -inf
included.

The order (the pages do not spell it out; this is the reading taken):
value descending, then token id ascending; every NaN ranks below -inf;
-0 and +0 are equal.  The returned values are the input's bits unchanged.
The sort is Python's (a library primitive) on that key.
"""

from __future__ import annotations

import math

import numpy as np


def order_key(v: float, j: int):
    """Sort key: smaller key = earlier in the pool."""
    v = float(v)
    if math.isnan(v):
        return (1, 0.0, j)
    return (0, -v if v != 0.0 else 0.0, j)


def topk_row(row: np.ndarray, K: int):
    """(values fp32 [K'], ids int32 [K']) with K' = min(K, len(row))."""
    row = np.asarray(row, dtype=np.float32)
    order = sorted(range(len(row)), key=lambda j: order_key(row[j], j))[:K]
    idx = np.array(order, dtype=np.int32)
    return row[idx].copy(), idx


def topk_rows(x: np.ndarray, K: int):
    vals, ids = zip(*(topk_row(r, K) for r in np.asarray(x, dtype=np.float32)))
    return np.stack(vals), np.stack(ids)
