"""Oracle: multi-segment split of the key axis and the merge of partial results.

Test infrastructure only.

Follows [summary] Methodologie 3 (the Multi-Segment strategy: segments of the
reduction are processed in parallel and their partial results are then merged)
and [explainer] section 3.3 (inter-block merge). Each segment t produces, from a
fresh state, the triple (m_t, s_t, o~_t): its own maximum, its sum of
exp(x - m_t) and its unnormalised accumulator sum exp(x - m_t) v. The merge is
the commutative-monoid combination the fusion conditions guarantee
([summary] Methodologie 1):

    m = max_t m_t,  w_t = exp(m_t - m),  s = sum_t w_t s_t,
    o = sum_t w_t o~_t / s,  lse = m + ln s.

Readings where the pages are silent: segments are contiguous, ceil(L / nseg)
long, the last ones possibly shorter or empty; an empty segment is the identity
(m_t = -inf, s_t = 0, o~_t = 0), with w_t = 0 for it; a row with no keys at all
merges to o = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np


def segment_bounds(L: int, nseg: int) -> list[tuple[int, int]]:
    """Contiguous segments of length ceil(L / nseg) covering [0, L)."""
    if L < 0 or nseg < 1:
        raise ValueError("need L >= 0 and nseg >= 1")
    c = -(-L // nseg)
    return [(min(L, t * c), min(L, (t + 1) * c)) for t in range(nseg)]


def split_partials(q, k, v, scale, nseg: int):
    """Per-segment partials for q [R, D] against k, v [R, L, D] (one query row per R).

    Returns part_m [R, nseg], part_s [R, nseg], part_o [R, nseg, D] (unnormalised)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    sigma = float(np.float32(scale))
    R, L, _ = k.shape
    pm = np.full((R, nseg), -np.inf)
    ps = np.zeros((R, nseg))
    po = np.zeros((R, nseg, v.shape[2]))
    x = sigma * np.einsum("rd,rld->rl", q, k)
    for t, (a, b) in enumerate(segment_bounds(L, nseg)):
        if b == a:
            continue
        xs = x[:, a:b]
        mt = xs.max(axis=1)
        p = np.exp(xs - mt[:, None])
        pm[:, t] = mt
        ps[:, t] = p.sum(axis=1)
        po[:, t] = np.einsum("rl,rld->rd", p, v[:, a:b])
    return pm, ps, po


def merge_partials(part_m, part_s, part_o):
    """Merge per-segment partials: [R, T], [R, T], [R, T, D] -> (o [R, D], lse [R])."""
    pm = np.asarray(part_m, np.float64)
    ps = np.asarray(part_s, np.float64)
    po = np.asarray(part_o, np.float64)
    m = pm.max(axis=1)
    with np.errstate(invalid="ignore"):
        w = np.where(np.isneginf(pm), 0.0, np.exp(pm - m[:, None]))
    s = (w * ps).sum(axis=1)
    acc = (w[:, :, None] * po).sum(axis=1)
    empty = s == 0
    with np.errstate(invalid="ignore", divide="ignore"):
        o = np.where(empty[:, None], 0.0, acc / np.where(empty, 1.0, s)[:, None])
        lse = np.where(empty, -np.inf, m + np.log(np.where(empty, 1.0, s)))
    return o, lse


def decode_split_merge(q, k, v, scale, nseg: int):
    """Split into nseg segments and merge: q [B,H,D], k [B,H,L,D], v [B,H,L,Dv] -> (o [B,H,Dv], lse [B,H])."""
    q = np.asarray(q, np.float64)
    B, H, D = q.shape
    L, Dv = np.shape(v)[2], np.shape(v)[3]
    pm, ps, po = split_partials(q.reshape(B * H, D), np.reshape(k, (B * H, L, D)),
                                np.reshape(v, (B * H, L, Dv)), scale, nseg)
    o, lse = merge_partials(pm, ps, po)
    return o.reshape(B, H, Dv), lse.reshape(B, H)
