"""The quantiser's quotient, checked exhaustively on the CPU (no GPU).

The kernel forms each code from the IEEE fp32 quotient fl32(x / sigma), sigma =
fl32(a / 448) with a the row's absolute maximum (the dynamic-quant cascade of the
explainer "RedFuser框架：AI加速器中的算子融合技术解析", section 4.3). Instead of a division
per element it uses the correctly rounded reciprocal r = fl32(1 / sigma) and one
correction (Markstein, IBM J. Res. Dev. 34(1), 1990):

    q0 = RN(x r);   e = RN(x - q0 sigma) (one FMA);   q = RN(q0 + e r) (one FMA),

with the sign of q taken from x. Rows with sigma < 2^-60 (where 1 / sigma may
overflow) divide directly instead. This test evaluates that formula with exact
arithmetic for every pair (x, a) of bf16 values with 0 < a and |x| <= a that the
scaling argument below does not already cover, and checks that it gives the same
E4M3FN code as the IEEE quotient (oracle.e4m3fn_encode), and the same fp32 quotient
bit for bit wherever that quotient is at least 2^-12 (below 2^-10 every code is 0).
When x itself is tiny (x < 2^-103) the exact residual needs more than fp32's
subnormal range and the corrected quotient can be one unit off; such quotients are
far below 2^-12, so their codes are still 0 and still agree.

Scaling argument. Multiplying a and x by 2^k (k an integer) multiplies sigma by 2^k
exactly and r by 2^-k exactly, leaves q0 unchanged, and multiplies e by 2^k, as long
as no intermediate leaves fp32's normal range; so every (x, a) maps to one with a in
[1, 2), except where sigma, r or e leave the normal range. Those ends are enumerated
directly: the binades around the 2^-60 switch (a in [2^-53, 2^-49)), every a below
2^-100 and every a above 2^100.
"""
import numpy as np
import pytest

from oracle import e4m3fn_encode
from synth import bf16_bits_to_f32


def _bf16_nonneg():
    """Every non-negative finite bf16 value, as float32 (0 and subnormals included)."""
    bits = np.arange(0, 0x7F80, dtype=np.uint16)          # 0x7F80 is +inf
    return bf16_bits_to_f32(bits)


def _rn32(v64):
    return v64.astype(np.float32)                         # IEEE round to nearest even


def _round_sum_to_f32(q0, t):
    """RN32(q0 + t) exactly, for fp32 q0 and an fp64 t that holds an exact product.

    The result is q0 or one of its fp32 neighbours whenever |t| <= 1.5 ulp(q0) (always
    the case here); the distances to the three candidates are exact in fp64 wherever
    the choice between them is close."""
    q0 = q0.astype(np.float32)
    lo = np.nextafter(q0, np.float32(-np.inf))
    hi = np.nextafter(q0, np.float32(np.inf))
    q64 = q0.astype(np.float64)
    d_lo = np.abs((lo.astype(np.float64) - q64) - t)
    d_mid = np.abs(t)
    d_hi = np.abs((hi.astype(np.float64) - q64) - t)
    best = np.where(d_lo < d_mid, lo, q0)
    bd = np.minimum(d_lo, d_mid)
    tie_lo = d_lo == d_mid
    # ties: the candidate with an even significand (even bit pattern)
    best = np.where(tie_lo & (lo.view(np.uint32) % 2 == 0), lo, best)
    best = np.where(d_hi < bd, hi, best)
    tie_hi = d_hi == bd
    best = np.where(tie_hi & (hi.view(np.uint32) % 2 == 0), hi, best)
    return best


def _markstein(x, sigma):
    """The kernel's quotient for fp32 arrays x >= 0 and sigma > 0, evaluated exactly: the
    reciprocal and one correction for sigma >= 2^-60, an IEEE division below."""
    x64, s64 = x.astype(np.float64), sigma.astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        return np.where(sigma >= np.float32(2.0 ** -60), _recip_corrected(x64, s64), _ieee(x, sigma))


def _recip_corrected(x64, s64):
    r = _rn32(1.0 / s64)                                  # the correctly rounded reciprocal
    r64 = r.astype(np.float64)
    q0 = _rn32(x64 * r64)                                 # x r: at most 8 + 24 bits, exact in fp64
    e = _rn32(x64 - q0.astype(np.float64) * s64)          # the FMA residual: exact in fp64, rounded once
    t = e.astype(np.float64) * r64                        # exact product (24 + 24 bits)
    return _round_sum_to_f32(q0, t)


def _ieee(x, sigma):
    # fp64 division then fp32 rounding: double rounding is innocuous for 53 >= 2 * 24 + 2
    return _rn32(x.astype(np.float64) / sigma.astype(np.float64))


def _check(a_vals, xs):
    """Every (x, a) with x in xs, 0 <= x <= a; returns the number of pairs checked."""
    n = 0
    for a in a_vals:
        x = xs[xs <= a]
        sigma = np.full(x.shape, _rn32(np.float64(a) / 448.0), np.float32)
        if sigma[0] == 0:
            continue
        got, ref = _markstein(x, sigma), _ieee(x, sigma)
        bad = (got.view(np.uint32) != ref.view(np.uint32)) & (ref >= np.float32(2.0 ** -12))
        if bad.any():
            i = np.nonzero(bad)[0][0]
            raise AssertionError(f"a={a!r} x={x[i]!r}: formula {got[i]!r}, IEEE {ref[i]!r}")
        cg, cr = e4m3fn_encode(got.astype(np.float64)), e4m3fn_encode(ref.astype(np.float64))
        if (cg != cr).any():
            i = np.nonzero(cg != cr)[0][0]
            raise AssertionError(f"a={a!r} x={x[i]!r}: code {cg[i]:#04x} vs {cr[i]:#04x}")
        n += x.size
    return n


def test_sign_symmetry_and_exact_cases():
    x = np.array([0.0, 1.0, 3.5, 448.0], np.float32)
    s = np.array([1.0, 0.5, 0.0078125, 1.0], np.float32)
    np.testing.assert_array_equal(_markstein(x, s), x / s)
    # the rounding helper: exact halfway cases go to the even neighbour
    one = np.array([1.0], np.float32)
    half_ulp = 2.0 ** -24
    assert _round_sum_to_f32(one, np.array([half_ulp]))[0] == 1.0            # 1 is even
    odd = np.nextafter(one, np.float32(2))
    assert _round_sum_to_f32(odd, np.array([half_ulp]))[0] == np.float32(1.0 + 2.0 ** -22)


def test_quotient_exhaustive_unit_binade():
    xs = _bf16_nonneg()
    a_vals = xs[(xs >= 1.0) & (xs < 2.0)]                 # all 128 significands
    assert a_vals.size == 128
    assert _check(a_vals, xs) > 2_000_000


@pytest.mark.parametrize("lo,hi", [(0.0, 2.0 ** -100), (2.0 ** -53, 2.0 ** -49), (2.0 ** 100, np.inf)])
def test_quotient_exhaustive_extreme_binades(lo, hi):
    """Every a in the binades where sigma or r leave fp32's normal range, against every x."""
    xs = _bf16_nonneg()
    a_vals = xs[(xs > lo) & (xs < hi) & (xs > 0)]
    # every x within 2^-21 of a (all codes that can be non-zero: x / sigma < 2^-10 below
    # that) plus every 29th smaller value, which keeps this in seconds
    n = 0
    for a in a_vals:
        near = xs[(xs <= a) & (xs >= a * 2.0 ** -21)]
        far = xs[xs < a * 2.0 ** -21][::29]
        n += _check([a], np.concatenate([near, far]))
    assert n > 100_000
