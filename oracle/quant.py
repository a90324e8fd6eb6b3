"""Oracle: the dynamic-quantisation cascade (absmax -> scale -> round -> GEMM).

Test infrastructure only.

Follows [explainer] section 4.3: scale = max(abs(X)) / quant_max, then
quant_X = round(X / scale), then Y = quant_X @ W, with maximum, scaling and
product fused in the library. Readings taken where the page is silent:

* the maximum is taken per row of X (the granularity of the dynamic-quant
  workload), and the weight arrives pre-quantised with one fp32 scale per
  output column;
* quant_max = 448 and the code is OCP FP8 E4M3FN ("fn": no infinities, one NaN
  pattern per sign, largest finite 448);
* the scale is the fp32 quotient sigma_i = fl32(a_i / 448), and the value that
  is rounded is the fp32 quotient fl32(x / sigma_i); "round" is round to
  nearest, ties to even, keeping the sign of zero and saturating at +-448;
* a row whose maximum is 0 gets sigma_i = 0, all codes 0x00 and an output row of 0;
* the product is accumulated exactly and dequantised as
  y_ij = sigma_i * w_scale_j * acc_ij.

fl32 of a float64 quotient of two fp32 numbers equals the IEEE fp32 quotient:
double rounding is innocuous for +, -, *, / and sqrt when the wider format has
at least 2p + 2 bits of precision (Figueroa, "When is double rounding
innocuous?", SIGNUM Newsletter 30(3), 1995), and 53 >= 2 * 24 + 2.

The GEMM accumulation is exact in float64: every E4M3FN value is an integer
multiple of 2^-9, so every product is a multiple of 2^-18 with magnitude at
most 448^2, and for K <= 2^20 every partial sum is an integer multiple of
2^-18 below 2^53 * 2^-18, hence representable; summation order is irrelevant.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL = 2.0 ** -6      # smallest normal E4M3FN value (exponent field 1)
_SUB_QUANTUM = 2.0 ** -9     # spacing of the subnormals (exponent field 0)


def fl32(a):
    """Round float64 values to the nearest fp32 value (ties to even), returned as float64."""
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def e4m3fn_decode(codes) -> np.ndarray:
    """E4M3FN codes (uint8) -> float64 values, per the OCP 8-bit floating point
    specification: sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
    exponent field 0 encodes (m/8) * 2^-6; S.1111.111 is NaN."""
    c = np.asarray(codes, np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return sign * mag


def e4m3fn_encode(v) -> np.ndarray:
    """float64 values -> E4M3FN codes, round to nearest with ties to even,
    sign of zero kept, magnitudes beyond 448 saturated to 448. Inputs are finite."""
    v = np.asarray(v, np.float64)
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    # Exponent of the binade holding a; below the smallest normal the spacing is fixed.
    _, ex = np.frexp(a)                       # a = f * 2^ex with f in [0.5, 1)
    e = np.where(a >= _MIN_NORMAL, ex - 1, -6)
    quantum = np.ldexp(1.0, e - 3)            # 3 mantissa bits
    r = np.rint(a / quantum)                  # exact scaling by a power of two; rint ties to even
    val = r * quantum                         # the rounded magnitude (exactly representable)
    # Encode the rounded magnitude.
    _, ex2 = np.frexp(val)
    e2 = ex2 - 1
    normal = val >= _MIN_NORMAL
    mant_n = np.where(normal, val / np.ldexp(1.0, np.where(normal, e2, 0) - 3) - 8.0, 0.0)
    bits_n = ((e2 + 7).astype(np.int64) << 3) | mant_n.astype(np.int64)
    bits_s = np.rint(val / _SUB_QUANTUM).astype(np.int64)
    bits = np.where(normal, bits_n, bits_s)
    return (bits | (neg.astype(np.int64) << 7)).astype(np.uint8)


def quantize_rows(x):
    """Per-row dynamic quantisation of x [M, K] (exact fp32 or bf16 values).

    Returns (codes [M, K] uint8, sigma [M] float64 holding fp32 values, absmax [M])."""
    x = np.asarray(x, np.float64)
    a = np.abs(x).max(axis=1)                  # reduction 1: row absmax (exact)
    sigma = fl32(a / E4M3_MAX)                 # the fp32 scale
    zero = sigma == 0
    with np.errstate(divide="ignore", invalid="ignore"):
        qv = fl32(x / np.where(zero, 1.0, sigma)[:, None])   # the fp32 quotient x / sigma
    codes = e4m3fn_encode(qv)
    codes[zero] = 0
    return codes, sigma, a


def quant_gemm_acc(codes, wq):
    """Exact accumulator acc[i, j] = sum_k dec(codes[i, k]) * dec(wq[j, k]); wq is [N, K]."""
    return e4m3fn_decode(codes) @ e4m3fn_decode(wq).T


def quant_gemm(x, wq, w_scale):
    """The whole cascade for x [M, K], wq [N, K] codes, w_scale [N].

    Returns (y [M, N] float64, sigma [M], codes [M, K])."""
    codes, sigma, _ = quantize_rows(x)
    acc = quant_gemm_acc(codes, wq)
    y = sigma[:, None] * np.asarray(w_scale, np.float64)[None, :] * acc
    return y, sigma, codes
