"""Pins for the MoE gate oracle (gate GEMM -> top-k -> softmax over the k)."""
from fractions import Fraction
import math

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from synth import bf16_bits_to_f32, moe_inputs


def _brute(x, w, k):
    """Exact rational scores, experts ordered by Python's sort on (-score, index),
    weights exp(s_r) / sum exp(s_r') evaluated with math.fsum."""
    T, Hd = x.shape
    E = w.shape[1]
    idx = np.zeros((T, k), np.int32)
    wt = np.zeros((T, k))
    for t in range(T):
        s = [sum(Fraction(float(x[t, h])) * Fraction(float(w[h, e])) for h in range(Hd)) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-s[e], e))[:k]
        idx[t] = order
        sf = [float(s[e]) for e in order]
        ex = [math.exp(v) for v in sf]
        tot = math.fsum(ex)
        wt[t] = [v / tot for v in ex]
    return idx, wt


@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 5), Hd=st.integers(1, 6), E=st.integers(1, 6), data=st.data(),
       seed=st.integers(0, 2**31 - 1), ints=st.booleans())
def test_brute_force_tiny(T, Hd, E, data, seed, ints):
    k = data.draw(st.integers(1, E))
    g = np.random.default_rng(seed)
    if ints:   # small integers make exact ties likely: the tie rule is exercised
        x = g.integers(-2, 3, (T, Hd)).astype(np.float64)
        w = g.integers(-2, 3, (Hd, E)).astype(np.float64)
    else:
        x = g.standard_normal((T, Hd)); w = g.standard_normal((Hd, E))
    idx, wt, _ = oracle.moe_route(x, w, k)
    bi, bw = _brute(x, w, k)
    if ints:
        np.testing.assert_array_equal(idx, bi)
    else:   # fp64 matmul vs exact rationals can only differ on near-ties, which random normals avoid
        np.testing.assert_array_equal(idx, bi)
    np.testing.assert_allclose(wt, bw, rtol=1e-13, atol=1e-15)


def test_lexsort_cross_check():
    g = np.random.default_rng(1)
    x = g.integers(-3, 4, (200, 8)).astype(np.float64)
    w = g.integers(-2, 3, (8, 12)).astype(np.float64)
    idx, _, s = oracle.moe_route(x, w, 4)
    ref = np.array([np.lexsort((np.arange(12), -row))[:4] for row in s])
    np.testing.assert_array_equal(idx, ref)


def test_k1_is_argmax():
    g = np.random.default_rng(2)
    x, w = g.standard_normal((300, 16)), g.standard_normal((16, 9))
    idx, wt, s = oracle.moe_route(x, w, 1)
    np.testing.assert_array_equal(idx[:, 0], np.argmax(s, axis=1))
    np.testing.assert_array_equal(wt, 1.0)


def test_top2_weights_logistic():
    g = np.random.default_rng(3)
    x, w = g.standard_normal((100, 32)), g.standard_normal((32, 16))
    idx, wt, s = oracle.moe_route(x, w, 2)
    s1 = np.take_along_axis(s, idx[:, :1], 1)[:, 0]
    s2 = np.take_along_axis(s, idx[:, 1:], 1)[:, 0]
    np.testing.assert_allclose(wt.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(wt[:, 0] >= 0.5)
    np.testing.assert_allclose(wt[:, 0], 1.0 / (1.0 + np.exp(s2 - s1)), rtol=1e-14)


def test_ties_resolve_to_lower_index():
    x = np.ones((1, 2))
    w = np.zeros((2, 6)); w[:, [1, 3, 4]] = 1.0   # experts 1, 3 and 4 tie at the top
    idx, wt, _ = oracle.moe_route(x, w, 2)
    np.testing.assert_array_equal(idx, [[1, 3]])
    np.testing.assert_allclose(wt, [[0.5, 0.5]], rtol=0, atol=0)


def test_column_permutation_permutes_indices():
    g = np.random.default_rng(4)
    x, w = g.standard_normal((64, 16)), g.standard_normal((16, 10))
    perm = g.permutation(10)
    idx, wt, _ = oracle.moe_route(x, w, 3)
    idx2, wt2, _ = oracle.moe_route(x, w[:, perm], 3)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(perm[idx2], idx)
    np.testing.assert_array_equal(inv[idx], idx2)
    np.testing.assert_allclose(wt2, wt, rtol=1e-13, atol=1e-15)


def test_generator_rejects_near_ties():
    x, w = moe_inputs(96, 64, 16, 2, seed=5, gap=0.05)
    s = bf16_bits_to_f32(x).astype(np.float64) @ bf16_bits_to_f32(w).astype(np.float64)
    top = -np.sort(-s, axis=1)[:, :3]
    assert np.all(top[:, 0] - top[:, 1] >= 0.05) and np.all(top[:, 1] - top[:, 2] >= 0.05)
    x2, w2 = moe_inputs(96, 64, 16, 2, seed=5, gap=0.05)
    np.testing.assert_array_equal(x, x2)
    np.testing.assert_array_equal(w, w2)
