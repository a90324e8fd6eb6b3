"""Oracle: the safe-softmax -> GEMM cascade (attention). Test infrastructure only.

Definition followed ([explainer] section 2.2, the softmax example; [summary],
Methodologie 1): three cascaded reductions over the key axis j of the scaled
scores x_j = sigma * <q, k_j>:

    reduction 1   m = max_j x_j
    reduction 2   s = sum_j exp(x_j - m)
    reduction 3   o = sum_j (exp(x_j - m) / s) * v_j

and lse = m + ln(s) (natural log of the scaled scores; the pages do not name
this output, it is the usual by-product of the first two reductions).

`attention_incremental` is the incremental (online) form that [explainer]
section 2.3 and [summary] Methodologie 2 describe: the key axis is consumed in
consecutive segments while only the running triple (m, s, o~) is kept. It is
used only to check that the incremental form and the three-pass definition
agree; it is written in its mathematically correct form (the old running sum
and accumulator are rescaled by exp(m_old - m_new); normalisation happens once
at the end), which is the reading taken where the explainer's section 4.1
pseudocode omits those factors.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _sigma(scale) -> float:
    # The scale is an fp32 argument of the library; the oracle uses that exact value.
    return float(np.float32(scale))


def attention(q, k, v, scale):
    """Three-pass softmax(sigma * Q K^T) V in float64.

    q [..., Sq, D], k and v [..., Sk, D] (Sk >= 1). Returns (o [..., Sq, D], lse [..., Sq]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    x = _sigma(scale) * np.matmul(q, np.swapaxes(k, -1, -2))     # scores [..., Sq, Sk]
    m = x.max(axis=-1, keepdims=True)                           # reduction 1: max
    p = np.exp(x - m)
    s = p.sum(axis=-1, keepdims=True)                           # reduction 2: sum of exp
    o = np.matmul(p / s, v)                                     # reduction 3: weighted sum of V
    lse = (m + np.log(s))[..., 0]
    return o, lse


def attention_incremental(q, k, v, scale, bounds):
    """The incremental form over consecutive key segments `bounds` = [(a, b), ...].

    The segments must tile [0, Sk) in order; empty segments leave the state
    unchanged. Returns (o, lse) like `attention`.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    sigma = _sigma(scale)
    lead = q.shape[:-1]
    m = np.full(lead, -np.inf)
    s = np.zeros(lead)
    o = np.zeros(lead + (v.shape[-1],))
    end = 0
    for a, b in bounds:
        if a != end:
            raise ValueError("segments must be consecutive")
        end = b
        if b == a:
            continue
        x = sigma * np.matmul(q, np.swapaxes(k[..., a:b, :], -1, -2))
        m_new = np.maximum(m, x.max(axis=-1))
        # alpha rescales the state built against the old maximum; a state that
        # has seen nothing yet (m = -inf) contributes nothing.
        with np.errstate(invalid="ignore"):
            alpha = np.where(np.isneginf(m), 0.0, np.exp(m - m_new))
        p = np.exp(x - m_new[..., None])
        s = alpha * s + p.sum(axis=-1)
        o = alpha[..., None] * o + np.matmul(p, v[..., a:b, :])
        m = m_new
    if end != k.shape[-2]:
        raise ValueError("segments must cover the key axis")
    return o / s[..., None], m + np.log(s)


def decode(q, k, v, scale):
    """One query token per (batch, head): q [B,H,D], k and v [B,H,L,D].

    Returns (o [B,H,D], lse [B,H]); identical to `attention` with Sq = 1."""
    o, lse = attention(_f64(q)[..., None, :], k, v, scale)
    return o[..., 0, :], lse[..., 0]


def decode_streaming(q_bh, kv_of, heads, scale):
    """`decode` for inputs too large to hold in float64 at once.

    q_bh(b, h) -> q [D]; kv_of(b, h) -> (k [L,D], v [L,D]); heads is an iterable
    of (b, h). Yields ((b, h), o [D], lse) one head at a time."""
    for b, h in heads:
        k, v = kv_of(b, h)
        o, lse = attention(_f64(q_bh(b, h))[None, :], k, v, scale)
        yield (b, h), o[0], float(lse[0])


def mla_decode(q, kv, d_v, scale):
    """Multi-head latent attention decode with the key projection absorbed ([summary],
    Resultaten, names MLA among the attention workloads): every head of batch entry b
    attends to the same cache rows, the keys are the whole rows and the values their
    first d_v entries. This is the plain definition above with the heads as the query rows.

    q [B, H, Dk], kv [B, L, Dk] (Dk >= d_v). Returns (o [B, H, d_v], lse [B, H])."""
    kv = _f64(kv)
    return attention(_f64(q), kv, kv[..., :d_v], scale)
