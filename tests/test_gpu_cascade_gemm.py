"""GPU parity: rf_cascade_gemm (the row-scaled GEMM cascades the generic template runs on
the matrix cores) against the plain definitions in oracle/cascade.py. Inputs are fp32 x and
bf16 W with fp32 accumulation: y and the softmax's logsumexp within 2e-2 + 1e-2 |r|, and,
from the arithmetic (each weight carried as two bf16 parts, |error| <= 2^-17 |p|, plus
fp32 accumulation over K terms), y within 2^-14 sum_k |p_k w_k| + 1e-6; the absolute
maximum bit-exact."""
import numpy as np
import pytest
import torch

from oracle import cascade
from synth import bf16_bits_to_f32, f32_to_bf16_bits
from tests.gpu_util import assert_close, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2
SHAPES = [(1, 4, 64), (5, 36, 128), (127, 100, 64), (128, 4096, 128), (300, 1000, 64), (1000, 64, 128),
          (129, 2052, 64), (33, 12, 128)]


def _inputs(M, K, N, seed, scale=3.0):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((M, K)) * scale).astype(np.float32)
    wb = f32_to_bf16_bits(g.standard_normal((K, N)).astype(np.float32))
    return x, wb


def _tight(y, ry, x, wb, kind):
    """|y - ref| <= 2^-14 sum_k |p_k| |w_k| + 1e-6 elementwise, p the exact weights."""
    w = np.abs(bf16_bits_to_f32(wb).astype(np.float64))
    xd = x.astype(np.float64)
    if kind == "softmax":
        m = xd.max(axis=1, keepdims=True)
        e = np.exp(xd - m)
        p = e / e.sum(axis=1, keepdims=True)
    else:
        a = np.abs(xd).max(axis=1, keepdims=True)
        p = np.abs(xd) / np.where(a == 0, 1.0, a)
    bound = 2.0 ** -14 * (p @ w) + 1e-6
    err = np.abs(y - ry)
    assert (err <= bound).all(), f"{int((err > bound).sum())} elements above the arithmetic bound"


def _run(rf, kind, x, wb):
    y, stat = rf.cascade_gemm(kind, dev_f32(x), dev_bf16(wb))
    torch.cuda.synchronize()
    return host(y), host(stat)


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_softmax_gemm(rf, M, K, N):
    x, wb = _inputs(M, K, N, 100 + M + K + N)
    y, lse = _run(rf, "softmax", x, wb)
    ry, rl = cascade.softmax_gemm(x, bf16_bits_to_f32(wb))
    assert_close(y, ry, ATOL, RTOL, "y")
    assert_close(lse, rl, ATOL, RTOL, "lse")
    _tight(y, ry, x, wb, "softmax")


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_absmax_gemm(rf, M, K, N):
    x, wb = _inputs(M, K, N, 200 + M + K + N, scale=1.0)
    x[np.random.default_rng(M).random(x.shape) < 0.01] *= 20          # 1% outliers
    y, a = _run(rf, "absmax", x, wb)
    ry, ra = cascade.absmax_gemm(x, bf16_bits_to_f32(wb))
    assert_close(y, ry, ATOL, RTOL, "y")
    _tight(y, ry, x, wb, "absmax")
    np.testing.assert_array_equal(a.astype(np.float32), ra.astype(np.float32))


def test_softmax_gemm_corrections_and_masks(rf):
    """Scores that grow along K (the lead moves in almost every chunk, so the output is
    corrected many times), large magnitudes, and -inf masks: a row masked except for one
    entry (y is that W row), a row whose first chunks are masked, every other chunk masked."""
    M, K, N = 64, 1024, 128
    x, wb = _inputs(M, K, N, 300)
    x[:16] += np.linspace(0, 60, K, dtype=np.float32)          # growing scores
    x[16:24] *= 40                                             # large magnitudes
    x[24, :] = -np.inf
    x[24, 777] = 5.0
    x[25, :200] = -np.inf
    for k0 in range(0, K, 64):
        x[26, k0:k0 + 32] = -np.inf
    y, lse = _run(rf, "softmax", x, wb)
    ry, rl = cascade.softmax_gemm(x, bf16_bits_to_f32(wb))
    assert np.isfinite(y).all() and np.isfinite(lse).all()
    assert_close(y, ry, ATOL, RTOL, "y")
    assert_close(lse, rl, ATOL, RTOL, "lse")
    np.testing.assert_array_equal(y[24], bf16_bits_to_f32(wb)[777].astype(np.float64))


def test_absmax_gemm_special_rows(rf):
    """A zero row (y = 0, stat = 0), a single non-zero, a negative extreme, |x| growing along
    K (a correction almost every chunk) and a row with W = I-like structure checked exactly."""
    M, K, N = 16, 640, 64
    x, wb = _inputs(M, K, N, 301, scale=1.0)
    x[0] = 0.0
    x[1] = 0.0
    x[1, 333] = -2.5
    x[2, 5] = -1000.0
    x[3] *= np.linspace(0.01, 50, K, dtype=np.float32)
    y, a = _run(rf, "absmax", x, wb)
    ry, ra = cascade.absmax_gemm(x, bf16_bits_to_f32(wb))
    assert_close(y, ry, ATOL, RTOL, "y")
    np.testing.assert_array_equal(a.astype(np.float32), ra.astype(np.float32))
    assert np.all(y[0] == 0) and a[0] == 0
    # a single non-zero: y = sign * that W row exactly (weight -1 is exact in bf16)
    np.testing.assert_array_equal(y[1], -bf16_bits_to_f32(wb)[333].astype(np.float64))


def test_deterministic(rf):
    x, wb = _inputs(300, 777 * 4, 128, 302)
    a = rf.cascade_gemm("softmax", dev_f32(x), dev_bf16(wb))
    b = rf.cascade_gemm("softmax", dev_f32(x), dev_bf16(wb))
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("kind", ["softmax", "absmax"])
@pytest.mark.parametrize("M,K,N", [(8200, 1000, 64), (4200, 100, 128)])
def test_many_workgroups_ragged_k(rf, kind, M, K, N):
    """Enough workgroups (of 128 rows) that they start their walk over K at different chunks,
    with a ragged last chunk that, at K = 100 (4 chunks), some workgroups meet first."""
    x, wb = _inputs(M, K, N, 400 + M + K, scale=3.0 if kind == "softmax" else 1.0)
    x[5, :] = -np.inf if kind == "softmax" else 0.0
    x[5, K - 1] = 2.0                                  # the only entry sits in the ragged chunk
    y, stat = _run(rf, kind, x, wb)
    ref = cascade.softmax_gemm if kind == "softmax" else cascade.absmax_gemm
    ry, rs = ref(x, bf16_bits_to_f32(wb))
    assert_close(y, ry, ATOL, RTOL, "y")
    _tight(y, ry, x, wb, kind)
    if kind == "softmax":
        assert_close(stat, rs, ATOL, RTOL, "lse")
        np.testing.assert_array_equal(y[5], bf16_bits_to_f32(wb)[K - 1].astype(np.float64))
    else:
        np.testing.assert_array_equal(stat.astype(np.float32), rs.astype(np.float32))


@pytest.mark.parametrize("kind", ["softmax", "absmax"])
def test_full_size_sampled(rf, kind):
    """The benchmarked shape, 65536 x 1024 fp32 against 1024 x 128 bf16, in the benchmarked
    launch; every 61st row (and the last) against the oracle."""
    M, K, N = 65536, 1024, 128
    x, wb = _inputs(M, K, N, 500, scale=3.0 if kind == "softmax" else 1.0)
    y, stat = _run(rf, kind, x, wb)
    rows = np.r_[np.arange(0, M, 61), M - 1]
    ref = cascade.softmax_gemm if kind == "softmax" else cascade.absmax_gemm
    ry, rs = ref(x[rows], bf16_bits_to_f32(wb))
    assert_close(y[rows], ry, ATOL, RTOL, "y")
    _tight(y[rows], ry, x[rows], wb, kind)
    if kind == "softmax":
        assert_close(stat[rows], rs, ATOL, RTOL, "lse")
    else:
        np.testing.assert_array_equal(stat[rows].astype(np.float32), rs.astype(np.float32))


_RNG_SHAPES = np.random.default_rng(4048)
RANDOM = [(int(_RNG_SHAPES.integers(1, 6000)), 4 * int(_RNG_SHAPES.integers(1, 700)),
           int(_RNG_SHAPES.choice([64, 128]))) for _ in range(8)]


@pytest.mark.parametrize("M,K,N", RANDOM)
def test_random_shapes(rf, M, K, N):
    """Seeded random shapes (up to 47 workgroups, so their walks over K start at different
    chunks, and K with or without a ragged last chunk), both kinds."""
    for kind, ref_fn, scale in (("softmax", cascade.softmax_gemm, 3.0), ("absmax", cascade.absmax_gemm, 1.0)):
        x, wb = _inputs(M, K, N, 600 + M + K + N, scale=scale)
        y, stat = _run(rf, kind, x, wb)
        ry, rs = ref_fn(x, bf16_bits_to_f32(wb))
        assert_close(y, ry, ATOL, RTOL, f"y ({kind})")
        _tight(y, ry, x, wb, kind)
        if kind == "softmax":
            assert_close(stat, rs, ATOL, RTOL, "lse")
        else:
            np.testing.assert_array_equal(stat.astype(np.float32), rs.astype(np.float32))
