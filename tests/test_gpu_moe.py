"""GPU parity: rf_moe_route against the oracle (gate GEMM -> top-k -> softmax).

Indices are compared bit-exactly. Random inputs come from the generator that
re-draws tokens with near-tied top scores (gap < 1e-2), so the top-k set and
order are unique under fp32 accumulation; exact ties are exercised with
integer-valued inputs, for which fp32 accumulation is exact."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, moe_inputs
from tests.gpu_util import assert_close, dev_bf16, host

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2


def _check(rf, x, w, k, check_scores=True, split=False):
    route = rf.moe_route_split if split else rf.moe_route
    idx, wt, sc = route(dev_bf16(x), dev_bf16(w), k, return_scores=check_scores)
    torch.cuda.synchronize()
    xf = bf16_bits_to_f32(x).astype(np.float64)
    wf = bf16_bits_to_f32(w).astype(np.float64)
    ridx, rw, rs = oracle.moe_route(xf, wf, k)
    gi = host(idx)
    np.testing.assert_array_equal(gi, ridx)
    assert_close(host(wt), rw, ATOL, RTOL, "weights")
    if check_scores:
        assert_close(host(sc), rs, ATOL, RTOL, "scores")
    return gi, host(wt)


@pytest.mark.parametrize("T,Hd,E,k", [
    (100, 256, 64, 2),     # ragged token block
    (1, 64, 16, 1),        # one token, smallest E
    (64, 4096, 64, 2),     # one token block, the full hidden size
    (130, 512, 256, 8),    # largest E and k
    (77, 1024, 48, 3),     # E not a power of two
    (300, 160, 32, 5),     # hidden size not a multiple of the range
    (50, 128, 128, 1),
    (20, 32, 16, 2),       # one hidden chunk: three of the four waves have none
    (40, 96, 64, 2),       # three chunks: one per wave, the last wave idle
    (9, 224, 80, 3),       # seven chunks: the last wave's chunk count is odd
    (1000, 2048, 64, 2),   # many workgroups
])
@pytest.mark.parametrize("split", [False, True], ids=["one_launch", "split"])
def test_route_shapes(rf, T, Hd, E, k, split):
    x, w = moe_inputs(T, Hd, E, k, seed=900 + T + E + k, w_std=0.5 if Hd < 1024 else 0.02)
    _check(rf, x, w, k, split=split)


def test_exact_ties_prefer_lower_index(rf):
    g = np.random.default_rng(3)
    T, Hd, E, k = 200, 64, 32, 4
    x = g.integers(-2, 3, (T, Hd)).astype(np.float32)
    w = g.integers(-1, 2, (Hd, E)).astype(np.float32)
    w[:, 20] = w[:, 3]          # experts 3 and 20 always tie
    w[:, 31] = w[:, 0]
    xb, wb = f32_to_bf16_bits(x), f32_to_bf16_bits(w)
    gi, _ = _check(rf, xb, wb, k)
    ties = 0
    for t in range(T):
        row = list(gi[t])
        if 3 in row and 20 in row:
            assert row.index(3) < row.index(20)
            ties += 1
    assert ties > 0


def test_repeated_calls_agree(rf):
    """Back-to-back calls agree bit for bit, and a smaller call after them is still right."""
    x, w = moe_inputs(256, 512, 64, 2, seed=31, w_std=0.5)
    a = _check(rf, x, w, 2, check_scores=False)
    b = _check(rf, x, w, 2, check_scores=False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    x2, w2 = moe_inputs(70, 256, 64, 2, seed=32, w_std=0.5)
    _check(rf, x2, w2, 2, check_scores=False)


@pytest.mark.parametrize("split", [False, True], ids=["one_launch", "split"])
def test_moe_workload(rf, split):
    """The routing workload: 2048 tokens x 4096 hidden, 64 experts, top-2."""
    c = CONFIGS["C4"]
    x, w = moe_inputs(c["T"], c["Hd"], c["E"], c["k"], c["seed"])
    _check(rf, x, w, c["k"], split=split)


def test_forms_agree(rf):
    """The one-launch and the two-launch forms select the same experts and agree on the weights."""
    x, w = moe_inputs(500, 1024, 64, 2, seed=33, w_std=0.02)
    a = _check(rf, x, w, 2, check_scores=False)
    b = _check(rf, x, w, 2, check_scores=False, split=True)
    assert np.array_equal(a[0], b[0])
    assert_close(b[1], a[1], 1e-5, 1e-5, "weights of the two forms")


_RNG_SHAPES = np.random.default_rng(77)
RANDOM = [(int(_RNG_SHAPES.integers(1, 600)), 32 * int(_RNG_SHAPES.integers(1, 160)),
           16 * int(_RNG_SHAPES.integers(1, 17)), int(_RNG_SHAPES.integers(1, 9))) for _ in range(8)]


@pytest.mark.parametrize("T,Hd,E,k", RANDOM)
@pytest.mark.parametrize("split", [False, True], ids=["one_launch", "split"])
def test_random_shapes(rf, T, Hd, E, k, split):
    """Seeded random token counts, hidden sizes, expert counts and k (indices bit-exact)."""
    k = min(k, E)
    x, w = moe_inputs(T, Hd, E, k, seed=1900 + T + E + k, w_std=0.5 if Hd < 1024 else 0.02)
    _check(rf, x, w, k, split=split)
