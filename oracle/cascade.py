"""Oracle: row cascades (the generic template's instances). Test infrastructure only.

Each function is the plain multi-pass definition of a cascade over the rows of
x [R, N] ([summary] Methodologie 1; [explainer] sections 2.1-2.2: a chain of
reductions where each one uses the results of the previous ones), in float64:

* logsumexp:        m = max_j x_j, then s = sum_j exp(x_j - m); lse = m + ln s;
* softmax_weighted: m, s as above, then o = sum_j exp(x_j - m) payload_j / s;
* topk_softmax:     the k best (score descending, index ascending), then the
                    softmax over those k (oracle.moe.topk_softmax);
* mean_var:         mu = mean_j x_j, then var = sum_j (x_j - mu)^2 / N
                    (population variance, the second reduction uses the first);
* softmax_gemm:     the softmax -> GEMM cascade with the scores given: per row of
                    x [M, K], m = max_k x_k, s = sum_k exp(x_k - m), then
                    y = sum_k exp(x_k - m) w_k / s against w [K, N], lse = m + ln s
                    ([explainer] sections 2.1 and 4.1);
* absmax_gemm:      a row-scaled GEMM: a = max_k |x_k|, then y = sum_k (x_k / a) w_k
                    (the dynamic-quant cascade of [explainer] section 4.3 without the
                    rounding); a row of zeros gives a = 0 and y = 0.
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


def softmax_gemm(x, w):
    """x [M, K] (scores; -inf entries are masked), w [K, N] -> (y [M, N], lse [M])."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    m = x.max(axis=1, keepdims=True)                 # reduction 1: the row maximum
    e = np.exp(x - m)
    s = e.sum(axis=1, keepdims=True)                 # reduction 2: uses reduction 1
    y = (e @ w) / s                                  # reduction 3: uses reductions 1 and 2
    return y, (m + np.log(s))[:, 0]


def absmax_gemm(x, w):
    """x [M, K], w [K, N] -> (y [M, N], a [M]) with a the row's absolute maximum."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    a = np.abs(x).max(axis=1)                        # reduction 1: the row's absolute maximum
    scaled = x / np.where(a == 0, 1.0, a)[:, None]   # a zero row stays zero
    return scaled @ w, a                             # reduction 2: uses reduction 1


__all__ = ["logsumexp", "softmax_weighted", "topk_softmax", "mean_var", "softmax_gemm", "absmax_gemm"]
