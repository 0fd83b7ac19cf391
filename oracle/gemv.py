"""Multi-row verify projection, the plain definition.

[SD] "Speculative decoding on RDNA", §01 "Why decode leaves room" and §02
"The draft is part of the model": one verify pass multiplies each weight
matrix by the k+1 verify rows at once; each row's result is the ordinary
single-row projection y = W x.

Weights are bf16 bit patterns (uint16), activations fp32.  The oracle
widens both exactly to fp64 and multiplies in fp64 (numpy matmul as the
primitive), which is exact to about 1e-16 relative for these sizes, and
also returns sum_k |w*x| per output, the scale of the parity tolerance.

Non-finite activations (the pages are silent; the plainest reading of the
sum): a row holding +-inf or NaN is evaluated term by term in IEEE fp64,
so an output is NaN if any term is NaN (a NaN activation, or an infinite
one times a zero weight) or if +inf and -inf terms meet, otherwise +-inf if
any term is infinite.  Subnormal activations are ordinary finite values.
Weights are model parameters and are taken to be finite.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> exact fp64 values (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def gemv_rows(w_bits: np.ndarray, x: np.ndarray, rows: np.ndarray | None = None,
              block: int = 8192):
    """Y[r][n] = sum_k W[n][k] * X[r][k] and S[r][n] = sum_k |W[n][k] * X[r][k]|.

    w_bits: uint16 [N][K]; x: float32 [R][K].  ``rows`` optionally selects
    output rows n (for spot checks of very large matrices).  Works in
    blocks of ``block`` output rows to bound memory.  Returns fp64 arrays
    Y, S of shape [R][len(rows) or N].
    """
    x64 = np.asarray(x, dtype=np.float32).astype(np.float64)
    idx = np.arange(w_bits.shape[0]) if rows is None else np.asarray(rows)
    R = x64.shape[0]
    y = np.empty((R, len(idx)), dtype=np.float64)
    s = np.empty((R, len(idx)), dtype=np.float64)
    ax = np.abs(x64)
    special = ~np.isfinite(x64).all(axis=1)  # rows evaluated term by term
    for b0 in range(0, len(idx), block):
        sel = idx[b0:b0 + block]
        w = bf16_bits_to_f64(w_bits[sel])
        with np.errstate(invalid="ignore"):
            y[:, b0:b0 + len(sel)] = x64 @ w.T
            s[:, b0:b0 + len(sel)] = ax @ np.abs(w).T
            for r in np.nonzero(special)[0]:
                terms = w * x64[r][None, :]              # [n][k], IEEE products
                y[r, b0:b0 + len(sel)] = terms.sum(axis=1)
                s[r, b0:b0 + len(sel)] = np.abs(terms).sum(axis=1)
    return y, s
