"""Oracle: the MoE gate cascade (gate GEMM -> top-k -> softmax). Test infrastructure only.

Follows [explainer] section 4.2: scores = x @ W_gate, then the top-k experts,
then a softmax that normalises the selected scores. Readings taken where the
page is silent:

* the order of the k outputs is descending score, equal scores ordered by the
  lower expert index (a stable sort on the negated score);
* the softmax runs over the k selected raw scores only (no temperature, bias
  or noise), i.e. top-k first, then softmax.
"""
from __future__ import annotations

import numpy as np


def gate_scores(x, w_gate):
    """S = X @ W_gate in float64: x [T, Hd], w_gate [Hd, E] -> [T, E]."""
    return np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64)


def topk_softmax(s, k: int):
    """The top-k -> softmax tail on given scores s [T, E]: returns (idx [T, k] int32, w [T, k])."""
    s = np.asarray(s, np.float64)
    E = s.shape[1]
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    order = np.argsort(-s, axis=1, kind="stable")   # ties keep the lower index first
    idx = order[:, :k]
    top = np.take_along_axis(s, idx, axis=1)
    e = np.exp(top - top[:, :1])                    # top[:, 0] is the largest selected score
    w = e / e.sum(axis=1, keepdims=True)
    return idx.astype(np.int32), w


def moe_route(x, w_gate, k: int):
    """Returns (idx [T, k] int32, w [T, k] float64, scores [T, E] float64)."""
    s = gate_scores(x, w_gate)
    idx, w = topk_softmax(s, k)
    return idx, w, s
