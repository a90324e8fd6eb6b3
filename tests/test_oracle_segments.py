"""Pins for the multi-segment split and the (max, sum, partial-O) merge oracle.

The merge is pinned by the commutative-monoid laws (commutativity,
associativity, identity of the empty segment) and by agreement of any split
with the unsplit three-pass attention.
"""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle


def test_segment_bounds_cover_and_ceil():
    for L in range(0, 40):
        for nseg in range(1, 12):
            b = oracle.segment_bounds(L, nseg)
            assert len(b) == nseg
            assert b[0][0] == 0 and b[-1][1] == L
            assert all(b[t][1] == b[t + 1][0] for t in range(nseg - 1))
            c = -(-L // nseg)
            assert all(e - s <= c for s, e in b)
            assert all(e - s == c for s, e in b[: L // c] if c) if L else True
    assert oracle.segment_bounds(10, 6) == [(0, 2), (2, 4), (4, 6), (6, 8), (8, 10), (10, 10)]
    with pytest.raises(ValueError):
        oracle.segment_bounds(5, 0)


@settings(max_examples=60, deadline=None)
@given(L=st.integers(1, 60), nseg=st.integers(1, 70), seed=st.integers(0, 2**31 - 1))
def test_split_merge_equals_unsplit(L, nseg, seed):
    g = np.random.default_rng(seed)
    q = g.standard_normal((2, 3, 8)) * 3
    k = g.standard_normal((2, 3, L, 8))
    v = g.standard_normal((2, 3, L, 5))
    o, lse = oracle.decode(q, k, v, 0.25)
    om, lsem = oracle.decode_split_merge(q, k, v, 0.25, nseg)
    np.testing.assert_allclose(om, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lsem, lse, rtol=1e-12, atol=1e-13)


def _partials(seed, R=4, T=7, D=3, empty=()):
    g = np.random.default_rng(seed)
    pm = g.standard_normal((R, T)) * 5
    ps = g.uniform(0.5, 40, (R, T))
    po = g.standard_normal((R, T, D)) * ps[..., None]
    for t in empty:
        pm[:, t], ps[:, t], po[:, t] = -np.inf, 0.0, 0.0
    return pm, ps, po


def test_merge_commutative():
    pm, ps, po = _partials(1)
    perm = np.random.default_rng(2).permutation(pm.shape[1])
    o, lse = oracle.merge_partials(pm, ps, po)
    o2, lse2 = oracle.merge_partials(pm[:, perm], ps[:, perm], po[:, perm])
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)


def test_merge_associative():
    pm, ps, po = _partials(3, T=9)
    o, lse = oracle.merge_partials(pm, ps, po)
    groups = [(0, 2), (2, 7), (7, 9)]
    # A merged group (o_g, lse_g) is itself a partial: maximum lse_g, sum 1, accumulator o_g.
    gm, gs, go = [], [], []
    for a, b in groups:
        og, lg = oracle.merge_partials(pm[:, a:b], ps[:, a:b], po[:, a:b])
        gm.append(lg); gs.append(np.ones_like(lg)); go.append(og)
    o2, lse2 = oracle.merge_partials(np.stack(gm, 1), np.stack(gs, 1), np.stack(go, 1))
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)


def test_merge_single_partial_is_normalisation():
    pm, ps, po = _partials(4, T=1)
    o, lse = oracle.merge_partials(pm, ps, po)
    np.testing.assert_allclose(o, po[:, 0] / ps[:, 0, None], rtol=1e-15)
    np.testing.assert_allclose(lse, pm[:, 0] + np.log(ps[:, 0]), rtol=1e-15)


def test_empty_partial_is_identity():
    pm, ps, po = _partials(5, T=6, empty=(1, 4))
    o, lse = oracle.merge_partials(pm, ps, po)
    keep = [0, 2, 3, 5]
    o2, lse2 = oracle.merge_partials(pm[:, keep], ps[:, keep], po[:, keep])
    np.testing.assert_allclose(o, o2, rtol=0, atol=0)
    np.testing.assert_allclose(lse, lse2, rtol=0, atol=0)


def test_all_empty_row():
    pm, ps, po = _partials(6, R=3, T=4)
    pm[1], ps[1], po[1] = -np.inf, 0.0, 0.0
    o, lse = oracle.merge_partials(pm, ps, po)
    assert np.all(o[1] == 0) and np.isneginf(lse[1])
    assert np.all(np.isfinite(o[[0, 2]])) and np.all(np.isfinite(lse[[0, 2]]))


def test_split_partials_match_brute_force():
    g = np.random.default_rng(7)
    q, k, v = g.standard_normal((2, 4)), g.standard_normal((2, 10, 4)), g.standard_normal((2, 10, 3))
    pm, ps, po = oracle.split_partials(q, k, v, 0.5, 4)    # segments of 3, 3, 3, 1
    for r in range(2):
        for t, (a, b) in enumerate([(0, 3), (3, 6), (6, 9), (9, 10)]):
            xs = [0.5 * float(np.dot(q[r], k[r, j])) for j in range(a, b)]
            mt = max(xs)
            assert pm[r, t] == pytest.approx(mt, rel=1e-15)
            assert ps[r, t] == pytest.approx(sum(np.exp(x - mt) for x in xs), rel=1e-14)
            np.testing.assert_allclose(po[r, t], sum(np.exp(xs[j - a] - mt) * v[r, j] for j in range(a, b)),
                                       rtol=1e-13)
