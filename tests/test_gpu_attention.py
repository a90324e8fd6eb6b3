"""GPU parity: rf_softmax_gemm_fused against the fp64 three-pass oracle."""
import numpy as np
import pytest

import oracle
from synth import CONFIGS, attn_inputs, bf16_bits_to_f32
from tests.gpu_util import assert_close, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu

F32_ATOL = 1e-5                 # fp32 inputs, fp32 accumulation
BF16_ATOL, BF16_RTOL = 2e-2, 1e-2


def _run(rf, inp):
    if inp.dtype == "f32":
        q, k, v = dev_f32(inp.q), dev_f32(inp.k), dev_f32(inp.v)
    else:
        q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    o, lse = rf.softmax_gemm_fused(q, k, v, inp.scale)
    import torch
    torch.cuda.synchronize()
    return host(o), host(lse)


def _ref(inp):
    if inp.dtype == "f32":
        return oracle.attention(inp.q, inp.k, inp.v, inp.scale)
    return oracle.attention(bf16_bits_to_f32(inp.q), bf16_bits_to_f32(inp.k), bf16_bits_to_f32(inp.v), inp.scale)


def test_f32_single_head_workload(rf):
    c = CONFIGS["C1"]
    inp = attn_inputs(c["B"], c["H"], c["Sq"], c["Sk"], c["D"], "f32", c["seed"], c["scale"])
    o, lse = _run(rf, inp)
    ro, rl = _ref(inp)
    assert_close(o, ro, F32_ATOL, 0.0, "O")
    assert_close(lse, rl, F32_ATOL, 0.0, "lse")


@pytest.mark.parametrize("B,H,Sq,Sk,D,scale", [
    (2, 3, 37, 300, 64, 0.125),     # ragged query and key tails, several key tiles per wave
    (1, 2, 5, 1, 64, 0.125),        # a single key
    (1, 1, 1, 17, 128, 0.0883883),  # one query row, D = 128
    (2, 1, 33, 129, 128, 0.5),      # ragged, D = 128
    (1, 1, 16, 2048, 64, 1.0),      # long key axis with large scores
    (3, 1, 70, 96, 64, 0.0),        # scale 0: every output row is the mean of V
])
def test_f32_shapes(rf, B, H, Sq, Sk, D, scale):
    inp = attn_inputs(B, H, Sq, Sk, D, "f32", seed=100 + Sq + Sk, scale=scale)
    o, lse = _run(rf, inp)
    ro, rl = _ref(inp)
    assert_close(o, ro, F32_ATOL, 0.0, "O")
    # Each score carries the fp32 rounding of its D-term dot product, which grows with the
    # score, and lse inherits it (scale 1 over 2048 keys: lse = 36.2, 1.19e-5 off, three
    # fp32 ulps); hence the relative term.
    assert_close(lse, rl, F32_ATOL, 1e-6, "lse")


def test_f32_deterministic(rf):
    inp = attn_inputs(2, 2, 40, 200, 64, "f32", seed=7)
    o1, l1 = _run(rf, inp)
    o2, l2 = _run(rf, inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------------ bf16 (matrix cores)


@pytest.mark.parametrize("B,H,Sq,Sk,D,scale", [
    (1, 2, 64, 64, 64, 0.125),        # one tile
    (2, 3, 100, 300, 64, 0.125),      # ragged queries and keys, several tiles
    (1, 1, 1, 1, 64, 0.125),          # one query, one key
    (1, 2, 130, 65, 64, 1.0),         # key tail of one, large scores
    (2, 2, 77, 200, 128, 0.0883883),  # D = 128
    (1, 1, 40, 1000, 64, 3.0),        # scores up to ~50: the reference maximum must move
    (1, 1, 64, 128, 64, -0.125),      # negative scale
    (1, 1, 64, 96, 64, 0.0),          # scale 0: the mean of V
])
def test_bf16_shapes(rf, B, H, Sq, Sk, D, scale):
    inp = attn_inputs(B, H, Sq, Sk, D, "bf16", seed=500 + Sq + Sk, scale=scale)
    o, lse = _run(rf, inp)
    ro, rl = _ref(inp)
    assert_close(o, ro, BF16_ATOL, BF16_RTOL, "O")
    assert_close(lse, rl, BF16_ATOL, BF16_RTOL, "lse")


def test_bf16_growing_scores(rf):
    """Keys whose scores grow along the key axis force a rescale on every tile."""
    inp = attn_inputs(1, 2, 64, 640, 64, "bf16", seed=21, scale=0.125)
    from synth import f32_to_bf16_bits
    kf = bf16_bits_to_f32(inp.k) + np.linspace(0, 12, 640, dtype=np.float32)[None, None, :, None] * \
        np.sign(bf16_bits_to_f32(inp.q).mean(axis=2, keepdims=True))
    inp.k = f32_to_bf16_bits(kf.astype(np.float32))
    o, lse = _run(rf, inp)
    ro, rl = _ref(inp)
    assert_close(o, ro, BF16_ATOL, BF16_RTOL, "O")
    assert_close(lse, rl, BF16_ATOL, BF16_RTOL, "lse")


def test_bf16_bert_workload(rf):
    """The BERT-base prefill shape: 8 x 12 heads, 512 x 512, D = 64, every output checked."""
    c = CONFIGS["C2"]
    inp = attn_inputs(c["B"], c["H"], c["Sq"], c["Sk"], c["D"], "bf16", c["seed"], c["scale"])
    o, lse = _run(rf, inp)
    ro, rl = _ref(inp)
    assert_close(o, ro, BF16_ATOL, BF16_RTOL, "O")
    assert_close(lse, rl, BF16_ATOL, BF16_RTOL, "lse")


def test_bf16_deterministic(rf):
    inp = attn_inputs(2, 2, 100, 300, 64, "bf16", seed=8)
    o1, l1 = _run(rf, inp)
    o2, l2 = _run(rf, inp)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("Sk,D,scale", [
    (128, 64, 0.125),      # two steps per key half
    (192, 64, 0.125),      # three steps: remainder of the unrolled loop
    (384, 128, 0.0883883), # six steps: the longest remainder, D = 128
    (448, 64, 0.125),      # seven steps: one whole unrolled round, no remainder
    (832, 64, 0.125),      # thirteen steps: two rounds
    (1024, 64, 3.0),       # large scores: the exact path moves the reference
    (128, 64, 0.0),        # scale 0
    (256, 128, -0.25),     # negative scale, D = 128
])
def test_bf16_whole_tiles(rf, Sk, D, scale):
    """Key lengths that are multiples of 64 take the loop without tail handling."""
    inp = attn_inputs(2, 2, 70, Sk, D, "bf16", seed=900 + Sk + D, scale=scale)
    o, lse = _run(rf, inp)
    ro, rl = _ref(inp)
    assert_close(o, ro, BF16_ATOL, BF16_RTOL, "O")
    assert_close(lse, rl, BF16_ATOL, BF16_RTOL, "lse")


def test_bf16_stepped_scores(rf):
    """Tiles of 32 keys whose scores are shifted by a per-tile offset (in units of ln 2 after
    scaling): a tile a few units above the reference makes its probability sum exceed 2^8
    without any probability doing so, one far above forces a rescale, and tiles far below
    underflow."""
    from synth import f32_to_bf16_bits
    Sk, D = 512, 64
    inp = attn_inputs(1, 2, 64, Sk, D, "bf16", seed=23, scale=0.125)
    qf = bf16_bits_to_f32(inp.q)
    kf = bf16_bits_to_f32(inp.k).copy()
    offs = np.array([0, 5, 5, 7, -30, 12, 2, 14, 14, 9, 20, 0, 6, 6, 30, 1], np.float32)   # per 32-key tile
    # Shift every key of tile t so that each query's score moves by about offs[t] * ln 2:
    # add c * mean(q) direction, scaled so that scale * q . dk = offs[t] * ln(2) on average.
    qm = qf.mean(axis=2, keepdims=True)                      # [B,H,1,D]
    nrm = (qm ** 2).sum(axis=3, keepdims=True)
    for t, off in enumerate(offs):
        kf[:, :, 32 * t:32 * (t + 1), :] += qm * (off * np.log(2) / inp.scale / nrm)
    inp.k = f32_to_bf16_bits(kf.astype(np.float32))
    o, lse = _run(rf, inp)
    ro, rl = _ref(inp)
    assert_close(o, ro, BF16_ATOL, BF16_RTOL, "O")
    assert_close(lse, rl, BF16_ATOL, BF16_RTOL, "lse")


# ------------------------------------------------------------------ whole-row (non-incremental) form


def _run_mode(rf, inp, mode):
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    o, lse = rf.softmax_gemm_fused(q, k, v, inp.scale, mode=mode)
    import torch
    torch.cuda.synchronize()
    return host(o), host(lse)


@pytest.mark.parametrize("B,H,Sq,Sk,D,scale", [
    (1, 2, 64, 1, 64, 0.125),         # a single key
    (2, 3, 100, 17, 64, 0.125),       # one partial tile, ragged query blocks
    (1, 2, 130, 32, 128, 0.0883883),  # exactly one tile, D = 128
    (2, 2, 77, 33, 64, 1.0),          # two tiles, the second with one key
    (1, 1, 128, 200, 128, 0.0883883), # seven tiles, D = 128
    (2, 1, 40, 255, 64, 3.0),         # large scores
    (1, 2, 300, 256, 64, 0.125),      # the longest row the form takes
    (1, 1, 64, 96, 64, -0.125),       # negative scale
    (1, 1, 64, 70, 64, 0.0),          # scale 0: the mean of V
])
def test_bf16_whole_row(rf, B, H, Sq, Sk, D, scale):
    inp = attn_inputs(B, H, Sq, Sk, D, "bf16", seed=700 + Sq + Sk, scale=scale)
    o, lse = _run_mode(rf, inp, "whole_row")
    ro, rl = _ref(inp)
    assert_close(o, ro, BF16_ATOL, BF16_RTOL, "O")
    assert_close(lse, rl, BF16_ATOL, BF16_RTOL, "lse")


def test_bf16_modes_agree_below_threshold(rf):
    """Below 256 keys the automatic choice is the whole-row form; both forms match the oracle."""
    inp = attn_inputs(2, 4, 256, 192, 64, "bf16", seed=77, scale=0.125)
    ro, rl = _ref(inp)
    for mode in ("auto", "whole_row", "incremental"):
        o, lse = _run_mode(rf, inp, mode)
        assert_close(o, ro, BF16_ATOL, BF16_RTOL, f"O ({mode})")
        assert_close(lse, rl, BF16_ATOL, BF16_RTOL, f"lse ({mode})")
    a, _ = _run_mode(rf, inp, "auto")
    w, _ = _run_mode(rf, inp, "whole_row")
    assert np.array_equal(a, w)


# Seeded random shapes through the automatic mode (incremental or whole-row by key length).
_RNG_SHAPES = np.random.default_rng(512)
RANDOM_BF16 = [(int(_RNG_SHAPES.integers(1, 3)), int(_RNG_SHAPES.integers(1, 5)), int(_RNG_SHAPES.integers(1, 700)),
                int(_RNG_SHAPES.integers(1, 1200)), int(_RNG_SHAPES.choice([64, 128]))) for _ in range(8)]


@pytest.mark.parametrize("B,H,Sq,Sk,D", RANDOM_BF16)
def test_bf16_random_shapes(rf, B, H, Sq, Sk, D):
    inp = attn_inputs(B, H, Sq, Sk, D, "bf16", seed=900 + Sq + Sk + D, scale=float(1.0 / np.sqrt(D)))
    o, lse = _run(rf, inp)
    ro, rl = _ref(inp)
    assert_close(o, ro, BF16_ATOL, BF16_RTOL, "O")
    assert_close(lse, rl, BF16_ATOL, BF16_RTOL, "lse")
