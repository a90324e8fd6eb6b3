"""GPU parity: rf_row_cascade (the generic incremental template's instances) against the
plain multi-pass definitions in oracle/cascade.py. fp32 inputs and fp32 accumulation:
|g - r| <= 1e-5; top-k indices bit-exact."""
import numpy as np
import pytest
import torch

import oracle
from oracle import cascade
from tests.gpu_util import assert_close, dev_f32, host

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-5, 0.0       # fp32 inputs: 1e-5 absolute
SHAPES = [(1, 1), (5, 3), (3, 255), (4, 256), (2, 257), (64, 1000), (7, 4096), (2, 4099)]


def _x(R, N, seed, scale=3.0, shift=0.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((R, N)) * scale + shift).astype(np.float32)


@pytest.mark.parametrize("R,N", SHAPES)
def test_logsumexp(rf, R, N):
    x = _x(R, N, 10 + N)
    got = host(rf.row_cascade("logsumexp", dev_f32(x)))
    assert_close(got, cascade.logsumexp(x), ATOL, RTOL, "lse")


@pytest.mark.parametrize("R,N", SHAPES)
@pytest.mark.parametrize("P", [1, 2, 4, 8, 16])
def test_softmax_weighted(rf, R, N, P):
    x = _x(R, N, 20 + N + P)
    p = np.random.default_rng(21 + N).standard_normal((R, N, P)).astype(np.float32)
    got = host(rf.row_cascade("softmax_weighted", dev_f32(x), dev_f32(p)))
    assert_close(got, cascade.softmax_weighted(x, p), ATOL, RTOL, "o")


# Lanes per top-k row: 4 at N = 8, 255 and 256, 8 at 1000, 16 at 1500, 32 at 2048, 64 at 4099 and
# 8192 (the four-at-a-time fold where N % 4 == 0, single inserts otherwise; DPP merges up to 16
# lanes, LDS permutes above).
@pytest.mark.parametrize("R,N", [(5, 8), (3, 255), (9, 256), (64, 1000), (5, 1500), (3, 2048), (2, 4099), (2, 8192)])
@pytest.mark.parametrize("k", [1, 2, 5, 8])
def test_topk_softmax(rf, R, N, k):
    # Scores on a grid of 1/4: many exact ties, which must resolve to the lower index.
    x = (np.round(_x(R, N, 30 + N + k) * 4) / 4).astype(np.float32)
    w, idx = rf.row_cascade("topk_softmax", dev_f32(x), k=k)
    ri, rw = oracle.topk_softmax(x.astype(np.float64), k)
    np.testing.assert_array_equal(host(idx), ri)
    assert_close(host(w), rw, ATOL, RTOL, "w")



@pytest.mark.parametrize("R,N", [(4, 256), (3, 1000), (2, 4099)])
def test_topk_softmax_nan_never_enters(rf, R, N):
    """NaN scores rank nowhere: the result equals the oracle's on the row with each NaN
    replaced by -inf (every row keeps far more than k finite scores)."""
    x = _x(R, N, 35 + N)
    g = np.random.default_rng(36 + N)
    x[g.random((R, N)) < 0.1] = np.nan
    x[0, :8] = np.nan                          # the first stretch of every lane of row 0
    w, idx = rf.row_cascade("topk_softmax", dev_f32(x), k=8)
    ri, rw = oracle.topk_softmax(np.where(np.isnan(x), -np.inf, x).astype(np.float64), 8)
    np.testing.assert_array_equal(host(idx), ri)
    assert_close(host(w), rw, ATOL, RTOL, "w")


@pytest.mark.parametrize("N", [8, 256, 1000])
def test_topk_softmax_signed_zero_ties(rf, N):
    """+0 and -0 compare equal, so they tie and the lower index ranks first, whichever sign it
    carries (the rank key turns -0 into +0)."""
    x = np.full((2, N), -1.0, np.float32)
    x[0, 3], x[0, 5] = 0.0, -0.0
    x[1, 3], x[1, 5] = -0.0, 0.0
    w, idx = rf.row_cascade("topk_softmax", dev_f32(x), k=2)
    np.testing.assert_array_equal(host(idx), [[3, 5], [3, 5]])
    np.testing.assert_array_equal(host(w), np.full((2, 2), 0.5))

@pytest.mark.parametrize("R,N", SHAPES)
def test_mean_var(rf, R, N):
    x = _x(R, N, 40 + N, scale=3.0, shift=10.0)
    got = host(rf.row_cascade("mean_var", dev_f32(x)))
    assert_close(got, cascade.mean_var(x), ATOL, RTOL, "mean/var")


def test_deterministic(rf):
    x = dev_f32(_x(16, 5000, 50))
    a = rf.row_cascade("mean_var", x)
    b = rf.row_cascade("mean_var", x)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _masked(R, N, seed):
    """Scores with -inf (masked) stretches: row 0 is masked except for its last element,
    row 1 masks the first 64 elements (a whole first stretch for every lane of a small
    group), row 2 masks every other 16-element block, the rest are unmasked."""
    x = _x(R, N, seed)
    x[0, :-1] = -np.inf
    x[1, :64] = -np.inf
    for j0 in range(0, N, 32):
        x[2, j0:j0 + 16] = -np.inf
    return x


@pytest.mark.parametrize("R,N", [(4, 100), (4, 256), (3, 1000), (4, 4099)])
def test_logsumexp_masked(rf, R, N):
    x = _masked(R, N, 60 + N)
    got = host(rf.row_cascade("logsumexp", dev_f32(x)))
    assert np.isfinite(got).all()
    assert_close(got, cascade.logsumexp(x), ATOL, RTOL, "lse")


@pytest.mark.parametrize("R,N", [(4, 100), (4, 256), (3, 1000), (4, 4099)])
@pytest.mark.parametrize("P", [1, 4, 16])
def test_softmax_weighted_masked(rf, R, N, P):
    x = _masked(R, N, 70 + N + P)
    p = np.random.default_rng(71 + N).standard_normal((R, N, P)).astype(np.float32)
    got = host(rf.row_cascade("softmax_weighted", dev_f32(x), dev_f32(p)))
    assert np.isfinite(got).all()
    assert_close(got, cascade.softmax_weighted(x, p), ATOL, RTOL, "o")
    # the row masked except for its last element returns that element's payload
    np.testing.assert_array_equal(got[0], p[0, -1].astype(np.float64))


# The benchmarked workloads at full size, in the benchmarked launch: inputs drawn on the device
# from a seeded generator, every output computed, every 61st row (and the last) checked against
# the oracle on the host.
FULL = [("logsumexp", 16384, 16384, 0, 0), ("mean_var", 16384, 16384, 0, 0),
        ("softmax_weighted", 4096, 8192, 4, 0), ("topk_softmax", 262144, 256, 0, 8)]


@pytest.mark.slow
@pytest.mark.parametrize("kind,R,N,P,k", FULL)
def test_workload_full_size_sampled(rf, kind, R, N, P, k):
    g = torch.Generator(device="cuda")
    g.manual_seed(80 + R % 97)
    x = torch.randn(R, N, device="cuda", generator=g)
    pay = torch.randn(R, N, P, device="cuda", generator=g) if P else None
    got = rf.row_cascade(kind, x, pay, k=k)
    torch.cuda.synchronize()
    rows = torch.cat([torch.arange(0, R, 61), torch.tensor([R - 1])]).to("cuda")
    xs = host(x.index_select(0, rows)).astype(np.float32)
    if kind == "topk_softmax":
        w, idx = got
        ridx, rw = cascade.topk_softmax(xs.astype(np.float64), k)
        np.testing.assert_array_equal(host(idx.index_select(0, rows)), ridx)
        assert_close(host(w.index_select(0, rows)), rw, ATOL, RTOL, "w")
        return
    g_rows = host(got.index_select(0, rows))
    if kind == "logsumexp":
        ref = cascade.logsumexp(xs)
    elif kind == "mean_var":
        ref = cascade.mean_var(xs)
    else:
        ref = cascade.softmax_weighted(xs, host(pay.index_select(0, rows)).astype(np.float32))
    assert_close(g_rows, ref, ATOL, RTOL, kind)


# Seeded random shapes: row counts and widths drawn across the lane-group sizes (4 to 64),
# the aligned and unaligned paths, and the spread payload mapping's stretch counts.
_RNG_SHAPES = np.random.default_rng(2024)
RANDOM = [(int(_RNG_SHAPES.integers(1, 300)), int(_RNG_SHAPES.integers(1, 9000))) for _ in range(12)]


@pytest.mark.parametrize("R,N", RANDOM)
def test_random_shapes(rf, R, N):
    g = np.random.default_rng(R * 10007 + N)
    x = (g.standard_normal((R, N)) * 3).astype(np.float32)
    assert_close(host(rf.row_cascade("logsumexp", dev_f32(x))), cascade.logsumexp(x), ATOL, RTOL, "lse")
    assert_close(host(rf.row_cascade("mean_var", dev_f32(x))), cascade.mean_var(x), ATOL, RTOL, "mean/var")
    for P in (4, 8):
        p = g.standard_normal((R, N, P)).astype(np.float32)
        got = host(rf.row_cascade("softmax_weighted", dev_f32(x), dev_f32(p)))
        assert_close(got, cascade.softmax_weighted(x, p), ATOL, RTOL, f"o (P = {P})")
    k = int(min(8, N))
    w, idx = rf.row_cascade("topk_softmax", dev_f32(x), k=k)
    ri, rw = oracle.topk_softmax(x.astype(np.float64), k)
    np.testing.assert_array_equal(host(idx), ri)
    assert_close(host(w), rw, ATOL, RTOL, "w")
