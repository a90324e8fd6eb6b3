"""Pins for the dynamic-quantisation oracle (absmax -> scale -> round -> GEMM).

The E4M3FN codec is pinned by torch's float8_e4m3fn decode of all 256 codes,
by brute-force nearest-value search with ties-to-even (including every exact
midpoint), and by torch's fp32 -> float8_e4m3fn cast over all finite bf16
values in range. The fp32 quotients are pinned by an exact rational rounding
routine; the GEMM by exact rational accumulation; the whole quantiser by
scaling invariants and the W = I special case.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from synth import bf16_bits_to_f32, f32_to_bf16_bits, quant_inputs

# ------------------------------------------------------------------ independent helpers


def _round_fraction_to_f32(fr: Fraction) -> float:
    """Exact round-to-nearest-even of a rational to fp32 (normal and subnormal range)."""
    if fr == 0:
        return 0.0
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    ulp = Fraction(2) ** (e - 23)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * float(fl * ulp)


def _e4m3_table():
    """Non-negative finite E4M3FN values by code 0..126, decoded by torch."""
    codes = torch.arange(0, 127, dtype=torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


_TABLE = None


def _nearest_code(v: float) -> int:
    """Brute force: the code of the nearest finite E4M3FN value, ties to the even code,
    sign kept (also for zero), saturating at 448."""
    global _TABLE
    if _TABLE is None:
        _TABLE = _e4m3_table()
    a = min(abs(v), 448.0)
    d = np.abs(_TABLE - a)
    best = np.flatnonzero(d == d.min())
    code = int(best[0]) if best.size == 1 else int([c for c in best if c % 2 == 0][0])
    return code | (0x80 if np.signbit(v) else 0)


# ------------------------------------------------------------------ codec


def test_decode_all_codes_vs_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_decode(codes)
    nan = np.isnan(ref)
    np.testing.assert_array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    np.testing.assert_array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_golden_code_table():
    """Named E4M3FN values from the OCP 8-bit floating point specification."""
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "e4m3fn_named_values.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    for code_hex, value in rows:
        code = int(code_hex, 16)
        val = float.fromhex(value) if value.startswith(("0x", "-0x")) else float(value)
        got = oracle.e4m3fn_decode(np.array([code], np.uint8))[0]
        if np.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (code_hex, value, got)
            assert oracle.e4m3fn_encode(np.array([val]))[0] == code


def test_encode_midpoints_ties_to_even():
    tab = _e4m3_table()
    for c in range(0, 126):
        mid = (tab[c] + tab[c + 1]) / 2          # exact in float64
        even = c if c % 2 == 0 else c + 1
        for sgn in (1.0, -1.0):
            got = oracle.e4m3fn_encode(np.array([sgn * mid]))[0]
            assert got == (even | (0x80 if sgn < 0 else 0)), (c, mid)
            lo = np.nextafter(mid, 0.0)
            hi = np.nextafter(mid, np.inf)
            assert oracle.e4m3fn_encode(np.array([sgn * lo]))[0] == (c | (0x80 if sgn < 0 else 0))
            assert oracle.e4m3fn_encode(np.array([sgn * hi]))[0] == ((c + 1) | (0x80 if sgn < 0 else 0))


def test_encode_brute_force_random():
    g = np.random.default_rng(1)
    v = np.concatenate([
        g.uniform(-460, 460, 3000),
        g.standard_normal(2000) * 2.0 ** -7,      # subnormal range
        np.exp2(g.uniform(-12, 9, 2000)) * g.choice([-1, 1], 2000),
        [0.0, -0.0, 448.0, -448.0, 447.9, 464.0, 1e6, -1e6, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.0000001],
    ]).astype(np.float32).astype(np.float64)
    got = oracle.e4m3fn_encode(v)
    ref = np.array([_nearest_code(x) for x in v], np.uint8)
    np.testing.assert_array_equal(got, ref)


def test_encode_vs_torch_all_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f32(bits)
    keep = np.isfinite(vals) & (np.abs(vals) <= 448.0)
    vals = vals[keep]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3fn_encode(vals.astype(np.float64))
    np.testing.assert_array_equal(got, ref)


def test_encode_vs_torch_random_fp32():
    g = np.random.default_rng(2)
    vals = np.concatenate([g.uniform(-448, 448, 200000), g.standard_normal(200000) * 0.01]).astype(np.float32)
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3fn_encode(vals.astype(np.float64)), ref)


# ------------------------------------------------------------------ fp32 rounding of quotients


def test_fl32_quotients_exact_rational():
    g = np.random.default_rng(3)
    a = g.standard_normal(3000).astype(np.float32) * np.float32(30)
    b = np.abs(g.standard_normal(3000)).astype(np.float32) + np.float32(1e-3)
    got = oracle.fl32(a.astype(np.float64) / b.astype(np.float64))
    for x, y, r in zip(a, b, got):
        assert r == _round_fraction_to_f32(Fraction(float(x)) / Fraction(float(y)))
    # and it is IEEE fp32 division
    np.testing.assert_array_equal(got.astype(np.float32), a / b)


# ------------------------------------------------------------------ quantiser


def _brute_quantize(x):
    M, K = x.shape
    codes = np.zeros((M, K), np.uint8)
    sig = np.zeros(M)
    for i in range(M):
        a = max(abs(Fraction(float(v))) for v in x[i])
        s = _round_fraction_to_f32(a / 448)
        sig[i] = s
        for k in range(K):
            if s == 0:
                codes[i, k] = 0
                continue
            q = _round_fraction_to_f32(Fraction(float(x[i, k])) / Fraction(s))
            if q == 0 and x[i, k] < 0:
                q = -0.0
            codes[i, k] = _nearest_code(q)
    return codes, sig


@settings(max_examples=40, deadline=None)
@given(M=st.integers(1, 4), K=st.integers(1, 8), seed=st.integers(0, 2**31 - 1), spread=st.sampled_from([1.0, 1e3, 1e-4]))
def test_quantize_brute_force(M, K, seed, spread):
    g = np.random.default_rng(seed)
    x = bf16_bits_to_f32(f32_to_bf16_bits((g.standard_normal((M, K)) * np.where(g.random((M, K)) < 0.3, spread, 1.0))
                                          .astype(np.float32))).astype(np.float64)
    codes, sig, _ = oracle.quantize_rows(x)
    bc, bs = _brute_quantize(x)
    np.testing.assert_array_equal(sig, bs)
    np.testing.assert_array_equal(codes, bc)


def test_quantize_power_of_two_scaling():
    g = np.random.default_rng(4)
    x = bf16_bits_to_f32(f32_to_bf16_bits(g.standard_normal((16, 64)).astype(np.float32))).astype(np.float64)
    c0, s0, _ = oracle.quantize_rows(x)
    for e in (-20, -3, 5, 40):
        c1, s1, _ = oracle.quantize_rows(x * 2.0 ** e)
        np.testing.assert_array_equal(c1, c0)
        np.testing.assert_array_equal(s1, s0 * 2.0 ** e)


def test_quantize_absmax_maps_to_448_and_zero_row():
    g = np.random.default_rng(5)
    x = bf16_bits_to_f32(f32_to_bf16_bits(g.standard_normal((32, 100)).astype(np.float32))).astype(np.float64)
    x[7] = 0.0
    codes, sig, a = oracle.quantize_rows(x)
    for i in range(32):
        if i == 7:
            assert sig[i] == 0 and np.all(codes[i] == 0)
            continue
        j = np.argmax(np.abs(x[i]))
        assert codes[i, j] == (0xFE if x[i, j] < 0 else 0x7E)
        assert np.all((codes[i] & 0x7F) <= 0x7E)


def test_negative_values_rounding_to_zero_keep_sign():
    x = np.array([[448.0, -1e-4, 1e-4, -0.0, 0.0]])
    codes, sig, _ = oracle.quantize_rows(x)
    assert sig[0] == 1.0
    np.testing.assert_array_equal(codes[0], [0x7E, 0x80, 0x00, 0x80, 0x00])


# ------------------------------------------------------------------ GEMM


def test_gemm_exact_rational_tiny():
    g = np.random.default_rng(6)
    codes = g.integers(0, 256, (3, 10)).astype(np.uint8)
    wq = g.integers(0, 256, (4, 10)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C   # no NaN codes
    wq[(wq & 0x7F) == 0x7F] = 0x41
    acc = oracle.quant_gemm_acc(codes, wq)
    dec = {c: Fraction(float(torch.tensor([c], dtype=torch.uint8).view(torch.float8_e4m3fn).float()))
           for c in range(256) if (c & 0x7F) != 0x7F}
    for i in range(3):
        for j in range(4):
            assert acc[i, j] == float(sum(dec[int(codes[i, k])] * dec[int(wq[j, k])] for k in range(10)))


def test_gemm_identity_weight():
    g = np.random.default_rng(7)
    x = bf16_bits_to_f32(f32_to_bf16_bits(g.standard_normal((8, 32)).astype(np.float32))).astype(np.float64)
    wq = np.zeros((32, 32), np.uint8)
    np.fill_diagonal(wq, 0x38)             # 1.0
    y, sig, codes = oracle.quant_gemm(x, wq, np.ones(32, np.float32))
    np.testing.assert_array_equal(y, sig[:, None] * oracle.e4m3fn_decode(codes))
    # and the dequantised codes approximate x within half an fp8 step of the row scale
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -4 + sig[:, None] * 2.0 ** -10 + 1e-30)


def test_gemm_close_to_unquantised_product():
    x, wq, ws = quant_inputs(16, 24, 256, seed=8)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    y, _, _ = oracle.quant_gemm(xf, wq, ws)
    w_deq = oracle.e4m3fn_decode(wq) * ws.astype(np.float64)[:, None]
    ref = xf @ w_deq.T
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel < 0.05      # e4m3 has 3 mantissa bits: relative step 2^-4


def test_weight_generator_uses_row_absmax():
    _, wq, ws = quant_inputs(4, 20, 64, seed=9)
    for j in range(20):
        assert np.any((wq[j] & 0x7F) == 0x7E)    # the column absmax maps to 448
    assert ws.dtype == np.float32 and np.all(ws > 0)
