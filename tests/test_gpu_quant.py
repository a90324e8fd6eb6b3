"""GPU parity: rf_quant_gemm (two launches) and rf_quant_gemm_fused (one launch) against
the oracle (absmax -> scale -> round -> GEMM).

Row scales and E4M3FN codes must be bit-exact; Y is compared within the bf16
tolerance (the oracle accumulates exactly in fp64, the GPU in fp32 on the
matrix cores and rounds Y to bf16). The one-launch form must also reproduce the
two-launch form's Y, scales and codes bit for bit (same quantiser, same order of
products)."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, quant_inputs
from tests.gpu_util import assert_close, dev_bf16, dev_f32, dev_u8, host

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


FORMS = ["two_launch", "fused"]


def _check(rf, x, wq, ws, use_workspace=False, form="two_launch"):
    dx, dwq, dws = dev_bf16(x), dev_u8(wq), dev_f32(ws)
    if form == "fused":
        y, xs, codes = rf.quant_gemm_fused(dx, dwq, dws, return_codes=not use_workspace)
        y2, xs2, codes2 = rf.quant_gemm(dx, dwq, dws, return_codes=True)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "fused Y differs from the two-launch Y"
        assert torch.equal(xs, xs2), "fused scales differ"
        if codes is not None:
            assert torch.equal(codes, codes2), "fused codes differ"
    elif use_workspace:
        y, xs, _ = rf.quant_gemm(dx, dwq, dws)
        codes = None
    else:
        y, xs, codes = rf.quant_gemm(dx, dwq, dws, return_codes=True)
    torch.cuda.synchronize()
    xf = bf16_bits_to_f32(x).astype(np.float64)
    ry, rsig, rcodes = oracle.quant_gemm(xf, wq, ws)
    np.testing.assert_array_equal(host(xs).astype(np.float32), rsig.astype(np.float32))
    if codes is not None:
        gc = codes.cpu().numpy()
        bad = np.argwhere(gc != rcodes)
        assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: got {gc[tuple(bad[0])]:#x} " \
                              f"want {rcodes[tuple(bad[0])]:#x} (x={xf[tuple(bad[0])]!r})"
    assert_close(host(y), ry, ATOL, RTOL, "Y")
    return host(y)


@pytest.mark.parametrize("M,N,K", [
    (5, 7, 128),          # far below one tile
    (100, 300, 256),      # ragged tiles in both directions
    (256, 256, 512),      # exactly one tile
    (1, 1, 128),
    (300, 520, 1024),
    (513, 257, 384),
    (70, 90, 2048),       # four 8-value chunks per lane in the row quantiser
    (9, 33, 8192),        # sixteen chunks per lane: the longest rows kept in registers
])
@pytest.mark.parametrize("form", FORMS)
def test_quant_gemm_shapes(rf, M, N, K, form):
    x, wq, ws = quant_inputs(M, N, K, seed=700 + M + N + K)
    _check(rf, x, wq, ws, form=form)


@pytest.mark.parametrize("form", FORMS)
def test_zero_and_tiny_rows(rf, form):
    x, wq, ws = quant_inputs(40, 64, 256, seed=71)
    xf = bf16_bits_to_f32(x).copy()
    xf[3] = 0.0                                         # zero row: scale 0, codes 0, Y row 0
    xf[5] = xf[5] * np.float32(1e-30)                   # tiny magnitudes (subnormal-range quotients avoided)
    xf[7, :] = 0.0
    xf[7, 10] = -2.0                                    # a single nonzero: every other code is +0
    xf[9] = np.where(np.arange(256) % 2 == 0, 1e-3, -1e-3).astype(np.float32)
    xf[9, 0] = 40.0                                     # many values that round to +-0 (codes 0x00 / 0x80)
    x = f32_to_bf16_bits(xf.astype(np.float32))
    y = _check(rf, x, wq, ws, form=form)
    assert np.all(y[3] == 0)


@pytest.mark.parametrize("form", FORMS)
def test_extreme_row_magnitudes(rf, form):
    """Rows whose absolute maximum spans bf16's range: a bf16 subnormal absmax (the scale is an
    fp32 subnormal and its reciprocal would overflow), scales on both sides of the switch
    from reciprocal-and-correction to division at 2^-60, and large magnitudes. Codes and
    scales bit-exact."""
    x, wq, ws = quant_inputs(24, 64, 256, seed=74)
    xf = bf16_bits_to_f32(x).astype(np.float64)
    scales = [2.0 ** -140, 2.0 ** -133, 2.0 ** -128, 2.0 ** -120, 2.0 ** -100, 2.0 ** -62, 2.0 ** -59,
              2.0 ** -52, 2.0 ** -49, 2.0 ** 20, 2.0 ** 60, 2.0 ** 90]
    for i, sc in enumerate(scales):
        xf[i] = xf[i] * sc
    x = f32_to_bf16_bits(xf.astype(np.float32))
    _check(rf, x, wq, ws, form=form)


def test_workspace_path_matches(rf):
    x, wq, ws = quant_inputs(130, 200, 512, seed=72)
    a = _check(rf, x, wq, ws, use_workspace=False)
    b = _check(rf, x, wq, ws, use_workspace=True)
    c = _check(rf, x, wq, ws, use_workspace=True, form="fused")     # fused, codes not stored
    assert np.array_equal(a, b) and np.array_equal(a, c)


@pytest.mark.parametrize("form", FORMS)
def test_identity_weight(rf, form):
    """W = I (codes 0x38 = 1.0 on the diagonal, unit scales): Y = sigma_i * dec(c_ik)."""
    x, _, _ = quant_inputs(64, 256, 256, seed=73)
    wq = np.zeros((256, 256), np.uint8)
    np.fill_diagonal(wq, 0x38)
    _check(rf, x, wq, np.ones(256, np.float32), form=form)


@pytest.mark.slow
def test_quant_gemm_workload(rf):
    """The 4096^3 workload: every scale, every code and every output element checked."""
    c = CONFIGS["C5"]
    x, wq, ws = quant_inputs(c["M"], c["N"], c["K"], c["seed"])
    _check(rf, x, wq, ws)


@pytest.mark.slow
def test_quant_gemm_fused_workload(rf):
    """The 4096^3 workload in one launch: Y, scales and codes bit-identical to the two-launch
    form (which the test above checks against the oracle element by element), and a sample
    of 64 rows against the oracle directly."""
    c = CONFIGS["C5"]
    x, wq, ws = quant_inputs(c["M"], c["N"], c["K"], c["seed"])
    dx, dwq, dws = dev_bf16(x), dev_u8(wq), dev_f32(ws)
    y, xs, codes = rf.quant_gemm_fused(dx, dwq, dws, return_codes=True)
    y2, xs2, codes2 = rf.quant_gemm(dx, dwq, dws, return_codes=True)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(xs, xs2) and torch.equal(codes, codes2)
    rows = np.unique(np.concatenate([np.random.default_rng(5).choice(c["M"], 62, replace=False), [0, c["M"] - 1]]))
    xf = bf16_bits_to_f32(x[rows]).astype(np.float64)
    ry, rsig, rcodes = oracle.quant_gemm(xf, wq, ws)
    np.testing.assert_array_equal(host(xs)[rows].astype(np.float32), rsig.astype(np.float32))
    np.testing.assert_array_equal(codes.cpu().numpy()[rows], rcodes)
    assert_close(host(y)[rows], ry, ATOL, RTOL, "Y (sampled rows)")


def _all_finite_codes():
    c = np.arange(256, dtype=np.uint8)
    return c[(c & 0x7F) != 0x7F]                       # 254 codes: both zeros, subnormals, normals


@pytest.mark.parametrize("form", FORMS)
def test_every_code_through_the_activation_operand(rf, form):
    """X row 0 holds every finite E4M3FN value (absmax 448, so sigma = 1 and the codes
    are the values themselves); with W = I, Y row 0 must equal those values exactly."""
    codes = _all_finite_codes()
    vals = oracle.e4m3fn_decode(codes)
    K = 256
    xf = np.zeros((2, K), np.float32)
    xf[0, :codes.size] = vals
    xf[1, 0] = 1.0
    x = f32_to_bf16_bits(xf)
    wq = np.zeros((K, K), np.uint8)
    np.fill_diagonal(wq, 0x38)
    y = _check(rf, x, wq, np.ones(K, np.float32), form=form)
    np.testing.assert_array_equal(y[0, :codes.size], vals)


@pytest.mark.parametrize("form", FORMS)
def test_every_code_through_the_weight_operand(rf, form):
    """X = 448 I (each row's only nonzero is 448: sigma = 1, code 0x7E); W column j holds
    every finite code, so Y = 448 * dec(code), exact in bf16."""
    codes = _all_finite_codes()
    K = 256
    x = f32_to_bf16_bits((np.eye(K, dtype=np.float32) * 448.0))
    wq = np.zeros((4, K), np.uint8)
    wq[0, :codes.size] = codes
    wq[1, :codes.size] = codes[::-1]
    y = _check(rf, x, wq, np.ones(4, np.float32), form=form)
    np.testing.assert_array_equal(y[:codes.size, 0], 448.0 * oracle.e4m3fn_decode(codes))
    np.testing.assert_array_equal(y[:codes.size, 1], 448.0 * oracle.e4m3fn_decode(codes[::-1]))


@pytest.mark.parametrize("form", FORMS)
def test_midpoints_round_to_even(rf, form):
    """Rows with absmax 448 have sigma = 1, so x / sigma = x exactly: inputs at every
    midpoint between adjacent E4M3FN values (representable in bf16) must round to the
    even code, and values one bf16 step either side to the nearer one."""
    codes = np.arange(0, 126, dtype=np.uint8)
    lo, hi = oracle.e4m3fn_decode(codes), oracle.e4m3fn_decode(codes + 1)
    mids = (lo + hi) / 2
    rows = []
    for sgn in (1.0, -1.0):
        for delta in (0, -1, 1):
            mb = f32_to_bf16_bits((sgn * mids).astype(np.float32)).astype(np.int64)
            mb = (mb + delta * (1 if sgn > 0 else 1)).astype(np.uint16) if delta else mb.astype(np.uint16)
            row = np.zeros(128, np.float32)
            row[:mids.size] = bf16_bits_to_f32(mb)
            row[127] = 448.0
            rows.append(row)
    x = f32_to_bf16_bits(np.stack(rows))
    wq = np.zeros((16, 128), np.uint8)
    np.fill_diagonal(wq, 0x38)
    _check(rf, x, wq, np.ones(16, np.float32), form=form)     # codes compared bit-exactly with the oracle


@pytest.mark.parametrize("form", FORMS)
def test_long_rows_streaming_path(rf, form):
    """Rows longer than the 8192 values kept in registers are read twice."""
    x, wq, ws = quant_inputs(3, 5, 8448, seed=74)
    _check(rf, x, wq, ws, form=form)


@pytest.mark.parametrize("form", FORMS)
def test_signed_zero_inputs(rf, form):
    """-0.0 inputs keep their sign through the quotient: code 0x80 (IEEE -0 / sigma = -0)."""
    xf = np.zeros((4, 128), np.float32)
    xf[:, 0] = [1.0, -3.0, 200.0, -0.5]
    xf[:, 1::2] = -0.0
    x = f32_to_bf16_bits(xf)
    wq = np.zeros((8, 128), np.uint8)
    np.fill_diagonal(wq, 0x38)
    _check(rf, x, wq, np.ones(8, np.float32), form=form)


_RNG_SHAPES = np.random.default_rng(8)
RANDOM = [(int(_RNG_SHAPES.integers(1, 700)), int(_RNG_SHAPES.integers(1, 700)), 128 * int(_RNG_SHAPES.integers(1, 24)))
          for _ in range(6)]


@pytest.mark.parametrize("M,N,K", RANDOM)
@pytest.mark.parametrize("form", FORMS)
def test_random_shapes(rf, M, N, K, form):
    """Seeded random shapes (codes and scales bit-exact, both forms bit-identical)."""
    x, wq, ws = quant_inputs(M, N, K, seed=1700 + M + N + K)
    _check(rf, x, wq, ws, form=form)
