"""Pins for the row-cascade oracle (oracle/cascade.py): brute force on tiny rows with exact
or compensated arithmetic, and library routines that compute the same quantities."""
import math
from fractions import Fraction

import numpy as np
import scipy.special

import oracle
from oracle import cascade


def test_logsumexp_against_scipy_and_brute_force():
    g = np.random.default_rng(1)
    x = g.standard_normal((5, 37)) * 4
    np.testing.assert_allclose(cascade.logsumexp(x), scipy.special.logsumexp(x, axis=1), rtol=1e-14)
    row = [0.5, -1.25, 3.0]
    want = math.log(math.fsum(math.exp(v) for v in row))
    assert abs(cascade.logsumexp(np.array([row]))[0] - want) < 1e-15


def test_softmax_weighted_brute_force_and_closed_forms():
    g = np.random.default_rng(2)
    x = g.standard_normal((3, 6))
    p = g.standard_normal((3, 6, 2))
    got = cascade.softmax_weighted(x, p)
    for r in range(3):
        e = [math.exp(v) for v in x[r]]
        s = math.fsum(e)
        for c in range(2):
            assert abs(got[r, c] - math.fsum(e[j] * p[r, j, c] for j in range(6)) / s) < 1e-14
    # equal scores -> the mean payload; one dominant score -> that payload
    np.testing.assert_allclose(cascade.softmax_weighted(np.zeros((1, 4)), p[:1, :4]), p[:1, :4].mean(axis=1),
                               rtol=1e-14)
    xd = np.zeros((1, 6))
    xd[0, 4] = 1e3
    np.testing.assert_allclose(cascade.softmax_weighted(xd, p[:1]), p[:1, 4], rtol=1e-14)


def test_topk_softmax_against_lexsort_and_argmax():
    g = np.random.default_rng(3)
    s = np.round(g.standard_normal((40, 12)) * 2) / 2          # many exact ties
    idx, w = oracle.topk_softmax(s, 4)
    for t in range(40):
        order = np.lexsort((np.arange(12), -s[t]))            # score descending, index ascending
        np.testing.assert_array_equal(idx[t], order[:4])
        e = np.exp(s[t, order[:4]] - s[t, order[0]])
        np.testing.assert_allclose(w[t], e / e.sum(), rtol=1e-14)
    i1, w1 = oracle.topk_softmax(s, 1)
    np.testing.assert_array_equal(i1[:, 0], np.argmax(s, axis=1))
    np.testing.assert_array_equal(w1, 1.0)


def test_mean_var_exact_and_numpy():
    rows = [[1, 2, 4], [Fraction(1, 3), -2, Fraction(7, 2), 0, 5]]
    for row in rows:
        n = len(row)
        mu = sum(Fraction(v) for v in row) / n
        var = sum((Fraction(v) - mu) ** 2 for v in row) / n
        got = cascade.mean_var(np.array([[float(v) for v in row]]))[0]
        assert abs(got[0] - float(mu)) < 1e-15 and abs(got[1] - float(var)) < 1e-14
    g = np.random.default_rng(4)
    x = g.standard_normal((6, 1000)) * 3 + 10
    mv = cascade.mean_var(x)
    np.testing.assert_allclose(mv[:, 0], x.mean(axis=1), rtol=1e-14)
    np.testing.assert_allclose(mv[:, 1], x.var(axis=1), rtol=1e-12)
    # shift invariance of the variance, and a constant row
    np.testing.assert_allclose(cascade.mean_var(x + 1e3)[:, 1], mv[:, 1], rtol=1e-9)
    np.testing.assert_array_equal(cascade.mean_var(np.full((1, 9), 2.5)), [[2.5, 0.0]])
