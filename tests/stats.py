"""Chi-square goodness of fit of emitted tokens against a sparse distribution."""

import numpy as np
from scipy import stats


def chi2_pvalue(tokens, dist_ids, dist_probs, min_expected=5.0):
    """p-value that `tokens` were drawn from the distribution (ids, probs).

    Bins with expected count below `min_expected` are merged into one bin.
    A token outside the support gives p-value 0.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    n = len(tokens)
    if n == 0:
        return 1.0
    ids = np.asarray(dist_ids, dtype=np.int64)
    probs = np.asarray(dist_probs, dtype=np.float64)
    probs = probs / probs.sum()
    support = set(int(t) for t in ids)
    if any(int(t) not in support for t in np.unique(tokens)):
        return 0.0
    counts = np.array([(tokens == t).sum() for t in ids], dtype=np.float64)
    expected = probs * n
    big = expected >= min_expected
    obs = list(counts[big])
    exp = list(expected[big])
    if (~big).any():
        obs.append(counts[~big].sum())
        exp.append(expected[~big].sum())
    obs, exp = np.array(obs), np.array(exp)
    if len(obs) < 2:
        return 1.0
    stat = float(((obs - exp) ** 2 / exp).sum())
    return float(stats.chi2.sf(stat, len(obs) - 1))
