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


def test_softmax_gemm_brute_force():
    g = np.random.default_rng(5)
    x = g.standard_normal((3, 7)) * 3
    w = g.standard_normal((7, 5))
    y, lse = cascade.softmax_gemm(x, w)
    assert y.shape == (3, 5) and lse.shape == (3,)         # K != N != M: a transposed operand fails
    for i in range(3):
        e = [math.exp(v) for v in x[i]]                    # no maximum subtracted: another route
        s = math.fsum(e)
        for n in range(5):
            assert abs(y[i, n] - math.fsum(e[k] * w[k, n] for k in range(7)) / s) < 1e-13
        assert abs(lse[i] - math.log(s)) < 1e-14


def test_softmax_gemm_closed_forms_and_invariants():
    g = np.random.default_rng(6)
    x = g.standard_normal((4, 9)) * 2
    # w = I: the rows of y are the softmax rows; a column of ones in w gives 1
    y, _ = cascade.softmax_gemm(x, np.eye(9))
    np.testing.assert_allclose(y, scipy.special.softmax(x, axis=1), rtol=1e-14)
    w = g.standard_normal((9, 3))
    w1 = np.concatenate([w, np.ones((9, 1))], axis=1)
    y1, lse1 = cascade.softmax_gemm(x, w1)
    np.testing.assert_allclose(y1[:, 3], 1.0, rtol=1e-14)
    np.testing.assert_allclose(lse1, scipy.special.logsumexp(x, axis=1), rtol=1e-14)
    # equal rows of w: y is that row whatever x is
    v = g.standard_normal(3)
    yc, _ = cascade.softmax_gemm(x, np.tile(v, (9, 1)))
    np.testing.assert_allclose(yc, np.tile(v, (4, 1)), rtol=1e-13)
    # shift invariance: y unchanged, lse shifted by the same amount
    y0, l0 = cascade.softmax_gemm(x, w)
    ys, ls = cascade.softmax_gemm(x + 7.5, w)
    np.testing.assert_allclose(ys, y0, rtol=1e-12)
    np.testing.assert_allclose(ls, l0 + 7.5, rtol=1e-14)
    # masked scores (-inf) drop out: the same as the softmax over the unmasked columns
    xm = x.copy()
    xm[:, [1, 4]] = -np.inf
    ym, lm = cascade.softmax_gemm(xm, w)
    keep = [k for k in range(9) if k not in (1, 4)]
    yk, lk = cascade.softmax_gemm(x[:, keep], w[keep])
    np.testing.assert_allclose(ym, yk, rtol=1e-14)
    np.testing.assert_allclose(lm, lk, rtol=1e-14)


def test_absmax_gemm_brute_force_and_invariants():
    rows = [[Fraction(3), Fraction(-5), Fraction(1, 2)], [Fraction(0), Fraction(0), Fraction(0)]]
    w = [[Fraction(1), Fraction(2)], [Fraction(-1, 4), Fraction(3)], [Fraction(5), Fraction(-7)]]
    y, a = cascade.absmax_gemm(np.array([[float(v) for v in r] for r in rows]),
                               np.array([[float(v) for v in r] for r in w]))
    for i, r in enumerate(rows):
        amax = max(abs(v) for v in r)
        assert a[i] == float(amax)
        for n in range(2):
            want = sum((v / amax if amax else Fraction(0)) * w[k][n] for k, v in enumerate(r))
            assert abs(y[i, n] - float(want)) < 1e-15
    g = np.random.default_rng(7)
    x = g.standard_normal((5, 11))
    wm = g.standard_normal((11, 4))
    y0, a0 = cascade.absmax_gemm(x, wm)
    # positive scaling of a row leaves y unchanged; a sign flip negates it
    y2, a2 = cascade.absmax_gemm(x * 3.25, wm)
    np.testing.assert_allclose(y2, y0, rtol=1e-13)
    np.testing.assert_allclose(a2, a0 * 3.25, rtol=1e-15)
    y3, _ = cascade.absmax_gemm(-x, wm)
    np.testing.assert_allclose(y3, -y0, rtol=1e-15)
    # w = I: the scaled rows themselves, every entry in [-1, 1] and one of them +-1
    yi, _ = cascade.absmax_gemm(x, np.eye(11))
    np.testing.assert_allclose(yi, x / np.abs(x).max(axis=1, keepdims=True), rtol=1e-15)
    assert np.all(np.isclose(np.abs(yi).max(axis=1), 1.0))
