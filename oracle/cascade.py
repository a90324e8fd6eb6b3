"""Oracle: row cascades (the generic template's instances). Test infrastructure only.

Each function is the plain multi-pass definition of a cascade over the rows of
x [R, N] ([summary] Methodologie 1; [explainer] sections 2.1-2.2: a chain of
reductions where each one uses the results of the previous ones), in float64:

* logsumexp:        m = max_j x_j, then s = sum_j exp(x_j - m); lse = m + ln s;
* softmax_weighted: m, s as above, then o = sum_j exp(x_j - m) payload_j / s;
* topk_softmax:     the k best (score descending, index ascending), then the
                    softmax over those k (oracle.moe.topk_softmax);
* mean_var:         mu = mean_j x_j, then var = sum_j (x_j - mu)^2 / N
                    (population variance, the second reduction uses the first).
"""
from __future__ import annotations

import numpy as np

from .moe import topk_softmax


def logsumexp(x):
    x = np.asarray(x, np.float64)
    m = x.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(axis=1, keepdims=True)))[:, 0]


def softmax_weighted(x, payload):
    """x [R, N], payload [R, N, P] -> [R, P]."""
    x = np.asarray(x, np.float64)
    p = np.asarray(payload, np.float64)
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    s = e.sum(axis=1, keepdims=True)
    return np.einsum("rn,rnp->rp", e, p) / s


def mean_var(x):
    """[R, 2]: the mean, then the population variance around it."""
    x = np.asarray(x, np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).sum(axis=1, keepdims=True) / x.shape[1]
    return np.concatenate([mu, var], axis=1)


__all__ = ["logsumexp", "softmax_weighted", "topk_softmax", "mean_var"]
