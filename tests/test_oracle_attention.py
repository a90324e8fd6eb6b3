"""Pins for the attention oracle (three-pass safe softmax -> GEMM).

Nothing here re-types the oracle's formula. The oracle is checked against:
an independent high-precision route (Decimal, no max subtraction) on tiny
inputs; scipy's softmax / logsumexp; closed forms; invariants; and the
incremental form over random segmentations. Shapes are chosen non-square
(Sq != Sk != D) so a transposed operand cannot pass.
"""
from decimal import Decimal, getcontext
import math

import numpy as np
import pytest
import scipy.special as sps
from hypothesis import given, settings, strategies as st

import oracle
from synth import attn_inputs


def _decimal_attention(q, k, v, scale):
    """softmax(sigma q k^T) v with 60-digit decimals, as exp(x) / sum exp(x)
    (no maximum is subtracted: a different route to the same number)."""
    getcontext().prec = 60
    sig = Decimal(float(np.float32(scale)))
    Sq, D = q.shape
    Sk = k.shape[0]
    o = np.zeros((Sq, v.shape[1]))
    lse = np.zeros(Sq)
    for i in range(Sq):
        xs = [sig * sum(Decimal(float(q[i, d])) * Decimal(float(k[j, d])) for d in range(D)) for j in range(Sk)]
        es = [x.exp() for x in xs]
        tot = sum(es)
        for c in range(v.shape[1]):
            o[i, c] = float(sum(es[j] * Decimal(float(v[j, c])) for j in range(Sk)) / tot)
        lse[i] = float(tot.ln())
    return o, lse


@settings(max_examples=60, deadline=None)
@given(Sq=st.integers(1, 3), Sk=st.integers(1, 4), D=st.integers(1, 3), Dv=st.integers(1, 3),
       seed=st.integers(0, 2**31 - 1), scale=st.sampled_from([1.0, 0.125, 0.7071067811865476, 2.5]))
def test_brute_force_tiny(Sq, Sk, D, Dv, seed, scale):
    g = np.random.default_rng(seed)
    q = g.standard_normal((Sq, D)) * 2
    k = g.standard_normal((Sk, D)) * 2
    v = g.standard_normal((Sk, Dv))
    o, lse = oracle.attention(q, k, v, scale)
    ob, lseb = _decimal_attention(q, k, v, scale)
    np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, lseb, rtol=1e-12, atol=1e-13)


def test_scipy_cross_check():
    inp = attn_inputs(2, 3, 17, 40, 8, "f32", seed=11, scale=0.3)
    o, lse = oracle.attention(inp.q, inp.k, inp.v, inp.scale)
    x = np.float32(0.3).astype(np.float64) * np.einsum("bhid,bhjd->bhij", inp.q.astype(np.float64),
                                                        inp.k.astype(np.float64))
    ref_o = np.einsum("bhij,bhjd->bhid", sps.softmax(x, axis=-1), inp.v.astype(np.float64))
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, sps.logsumexp(x, axis=-1), rtol=1e-13, atol=1e-13)


def test_torch_cpu_cross_check():
    import torch
    inp = attn_inputs(1, 2, 9, 33, 16, "f32", seed=12, scale=0.25)
    o, _ = oracle.attention(inp.q, inp.k, inp.v, inp.scale)
    tq, tk, tv = (torch.from_numpy(a.astype(np.float64)) for a in (inp.q, inp.k, inp.v))
    ref = torch.softmax(0.25 * tq @ tk.transpose(-1, -2), dim=-1) @ tv
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-13)


# ------------------------------------------------------------------ closed forms

def test_single_key():
    g = np.random.default_rng(1)
    q, k, v = g.standard_normal((5, 4)), g.standard_normal((1, 4)), g.standard_normal((1, 3))
    o, lse = oracle.attention(q, k, v, 0.5)
    np.testing.assert_allclose(o, np.repeat(v, 5, axis=0), rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse, 0.5 * (q @ k[0]), rtol=1e-15)


def test_two_keys_logistic():
    g = np.random.default_rng(2)
    q, k, v = g.standard_normal((6, 3)), g.standard_normal((2, 3)), g.standard_normal((2, 5))
    o, _ = oracle.attention(q, k, v, 1.0)
    d = q @ k[0] - q @ k[1]
    w0 = 1.0 / (1.0 + np.exp(-d))        # logistic function of the score difference
    np.testing.assert_allclose(o, w0[:, None] * v[0] + (1 - w0)[:, None] * v[1], rtol=1e-13, atol=1e-14)


def test_equal_scores_give_mean():
    g = np.random.default_rng(3)
    q = np.zeros((4, 8))                 # every score is 0
    k, v = g.standard_normal((10, 8)), g.standard_normal((10, 3))
    o, lse = oracle.attention(q, k, v, 0.125)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (4, 1)), rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(lse, np.log(10.0), rtol=1e-15)


def test_scale_zero_gives_mean():
    g = np.random.default_rng(4)
    q, k, v = g.standard_normal((3, 5)), g.standard_normal((7, 5)), g.standard_normal((7, 2))
    o, _ = oracle.attention(q, k, v, 0.0)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (3, 1)), rtol=1e-13, atol=1e-15)


def test_dominant_key_selects_its_row():
    g = np.random.default_rng(5)
    q = np.ones((2, 4))
    k = g.standard_normal((9, 4)) * 0.1
    k[6] = 300.0                         # score 1200 against O(1) for the rest
    v = g.standard_normal((9, 3))
    o, lse = oracle.attention(q, k, v, 1.0)
    np.testing.assert_allclose(o, np.tile(v[6], (2, 1)), rtol=0, atol=1e-300)
    np.testing.assert_allclose(lse, 1200.0, rtol=1e-15)


# ------------------------------------------------------------------ invariants

def test_rows_sum_to_one():
    inp = attn_inputs(2, 2, 13, 29, 6, "f32", seed=21, scale=0.4)
    v = np.ones((2, 2, 29, 1))
    o, _ = oracle.attention(inp.q, inp.k, v, inp.scale)
    np.testing.assert_allclose(o, 1.0, rtol=0, atol=1e-14)


def test_constant_value_rows():
    inp = attn_inputs(1, 1, 8, 20, 4, "f32", seed=22)
    row = np.array([1.5, -2.0, 0.25, 7.0])
    v = np.broadcast_to(row, (1, 1, 20, 4))
    o, _ = oracle.attention(inp.q, inp.k, v, inp.scale)
    np.testing.assert_allclose(o, np.broadcast_to(row, o.shape), rtol=1e-14, atol=1e-14)


def test_shift_invariance():
    inp = attn_inputs(1, 3, 11, 23, 8, "f32", seed=23, scale=0.125)
    k0 = np.random.default_rng(7).standard_normal(8)
    o, lse = oracle.attention(inp.q, inp.k, inp.v, inp.scale)
    o2, lse2 = oracle.attention(inp.q, inp.k.astype(np.float64) + k0, inp.v, inp.scale)
    shift = 0.125 * (inp.q.astype(np.float64) @ k0)
    np.testing.assert_allclose(o2, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + shift, rtol=1e-12, atol=1e-12)


def test_key_permutation():
    inp = attn_inputs(1, 2, 7, 31, 5, "f32", seed=24)
    perm = np.random.default_rng(8).permutation(31)
    o, lse = oracle.attention(inp.q, inp.k, inp.v, inp.scale)
    o2, lse2 = oracle.attention(inp.q, inp.k[:, :, perm], inp.v[:, :, perm], inp.scale)
    np.testing.assert_allclose(o2, o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse2, lse, rtol=1e-14)


def test_query_rows_independent():
    inp = attn_inputs(1, 1, 9, 15, 4, "f32", seed=25)
    o, _ = oracle.attention(inp.q, inp.k, inp.v, inp.scale)
    o3, _ = oracle.attention(inp.q[:, :, 3:4], inp.k, inp.v, inp.scale)
    np.testing.assert_allclose(o3[:, :, 0], o[:, :, 3], rtol=0, atol=1e-15)


# ------------------------------------------------------------------ incremental form

@st.composite
def _segmentation(draw):
    L = draw(st.integers(1, 40))
    cuts = sorted(set(draw(st.lists(st.integers(0, L), max_size=8))))
    edges = [0] + cuts + [L]
    return L, list(zip(edges[:-1], edges[1:]))    # may contain empty segments


@settings(max_examples=80, deadline=None)
@given(seg=_segmentation(), seed=st.integers(0, 2**31 - 1), big=st.booleans())
def test_incremental_equals_three_pass(seg, seed, big):
    L, bounds = seg
    g = np.random.default_rng(seed)
    q = g.standard_normal((3, 6)) * (8.0 if big else 1.0)   # large scores stress the rescaling
    k = g.standard_normal((L, 6))
    v = g.standard_normal((L, 4))
    o, lse = oracle.attention(q, k, v, 0.5)
    oi, lsei = oracle.attention_incremental(q, k, v, 0.5, bounds)
    np.testing.assert_allclose(oi, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lsei, lse, rtol=1e-12, atol=1e-13)


def test_incremental_rejects_gaps():
    q = np.zeros((1, 2)); k = np.zeros((4, 2)); v = np.zeros((4, 2))
    with pytest.raises(ValueError):
        oracle.attention_incremental(q, k, v, 1.0, [(0, 2), (3, 4)])
    with pytest.raises(ValueError):
        oracle.attention_incremental(q, k, v, 1.0, [(0, 2)])


def test_decode_is_single_query_attention():
    g = np.random.default_rng(9)
    q, k, v = g.standard_normal((2, 3, 8)), g.standard_normal((2, 3, 50, 8)), g.standard_normal((2, 3, 50, 8))
    o, lse = oracle.decode(q, k, v, 0.35)
    for b in range(2):
        for h in range(3):
            ob, lb = _decimal_attention(q[b, h][None], k[b, h], v[b, h], 0.35) if b == 0 and h == 0 else \
                oracle.attention(q[b, h][None], k[b, h], v[b, h], 0.35)
            np.testing.assert_allclose(o[b, h], ob[0], rtol=1e-12, atol=1e-13)
            np.testing.assert_allclose(lse[b, h], lb[0], rtol=1e-12)
    streamed = {bh: (oo, ll) for bh, oo, ll in oracle.decode_streaming(
        lambda b, h: q[b, h], lambda b, h: (k[b, h], v[b, h]), [(1, 2), (0, 1)], 0.35)}
    np.testing.assert_allclose(streamed[(1, 2)][0], o[1, 2], rtol=0, atol=0)
    assert math.isclose(streamed[(0, 1)][1], lse[0, 1], rel_tol=0, abs_tol=0)


def test_mla_decode_brute_force():
    """MLA decode against a pure-Python loop: keys are whole cache rows, values their first d_v
    entries, shared by every head (math.fsum, exact exp ratios)."""
    import math
    g = np.random.default_rng(11)
    B, H, L, Dk, dv, scale = 2, 3, 5, 4, 3, 0.7
    q = g.standard_normal((B, H, Dk))
    kv = g.standard_normal((B, L, Dk))
    o, lse = oracle.mla_decode(q, kv, dv, scale)
    assert o.shape == (B, H, dv) and lse.shape == (B, H)
    for b in range(B):
        for h in range(H):
            x = [float(np.float32(scale)) * math.fsum(q[b, h, d] * kv[b, j, d] for d in range(Dk)) for j in range(L)]
            m = max(x)
            e = [math.exp(xi - m) for xi in x]
            s = math.fsum(e)
            for d in range(dv):
                assert abs(o[b, h, d] - math.fsum(e[j] * kv[b, j, d] for j in range(L)) / s) < 1e-12
            assert abs(lse[b, h] - (m + math.log(s))) < 1e-12


def test_mla_decode_rotary_part_only_scores():
    """The rotary columns (past d_v) only enter the scores: with queries that are zero there,
    any change to those cache columns leaves O and lse unchanged; with all-zero queries O is
    the mean latent row and lse = ln L."""
    g = np.random.default_rng(12)
    q = g.standard_normal((1, 2, 8))
    q[..., 5:] = 0.0
    kv = g.standard_normal((1, 6, 8))
    o1, l1 = oracle.mla_decode(q, kv, 5, 0.3)
    kv2 = kv.copy()
    kv2[..., 5:] = g.standard_normal((1, 6, 3)) * 100.0
    o2, l2 = oracle.mla_decode(q, kv2, 5, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    o0, lse0 = oracle.mla_decode(np.zeros_like(q), kv, 5, 0.3)
    np.testing.assert_allclose(o0[0, 0], kv[0, :, :5].mean(axis=0), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse0, np.log(6.0), rtol=1e-14)
