"""GPU parity: rf_attn_decode_split + rf_segment_merge against the oracle.

Partials are compared with the oracle's per-segment partials; merged outputs
with the unsplit three-pass definition (decode = attention with one query)."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, bf16_bits_to_f32, decode_inputs, decode_kv_slice, decode_q
from tests.gpu_util import assert_close, dev_bf16, dev_f32, host

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2          # bf16 inputs, fp32 accumulation (outputs)
P_ATOL, P_RTOL = 1e-4, 1e-4      # fp32 partial statistics


def _f(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _check_case(rf, B, H, L, D, nseg, seed, out_dtype=torch.bfloat16):
    q, k, v, scale = decode_inputs(B, H, L, D, seed)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    pm, ps, po = rf.attn_decode_split(dq, dk, dv, nseg, scale)
    o, lse = rf.segment_merge(pm, ps, po, out_dtype)
    torch.cuda.synchronize()
    qf, kf, vf = _f(q), _f(k), _f(v)
    rpm, rps, rpo = oracle.split_partials(qf.reshape(B * H, D), kf.reshape(B * H, L, D), vf.reshape(B * H, L, D),
                                          scale, nseg)
    assert_close(host(pm), rpm, P_ATOL, P_RTOL, "part_m")
    assert_close(host(ps), rps, P_ATOL, P_RTOL, "part_s")
    assert_close(host(po), rpo, P_ATOL, P_RTOL, "part_o")
    ro, rl = oracle.decode(qf, kf, vf, scale)
    assert_close(host(o).reshape(B, H, D), ro, ATOL, RTOL, "O")
    assert_close(host(lse).reshape(B, H), rl, ATOL, RTOL, "lse")
    return host(o)


@pytest.mark.parametrize("B,H,L,D,nseg", [
    (2, 3, 100, 128, 1),      # single segment
    (2, 3, 100, 128, 3),      # ragged segments (34, 34, 32)
    (2, 3, 100, 128, 8),
    (1, 2, 100, 128, 100),    # one key per segment
    (1, 1, 10, 128, 6),       # trailing empty segment (2, 2, 2, 2, 2, 0)
    (1, 1, 1, 128, 1),        # a single key
    (2, 2, 37, 64, 5),        # D = 64
    (1, 4, 1000, 128, 7),     # several loop iterations per segment, ragged tail
])
def test_split_merge_small(rf, B, H, L, D, nseg):
    _check_case(rf, B, H, L, D, nseg, seed=300 + L + nseg)


def test_fp32_output(rf):
    _check_case(rf, 1, 3, 257, 128, 4, seed=11, out_dtype=torch.float32)


def test_merge_edge_cases(rf):
    g = np.random.default_rng(5)
    R, T, D = 6, 9, 128
    pm = g.standard_normal((R, T)) * 4
    ps = g.uniform(0.5, 30, (R, T))
    po = g.standard_normal((R, T, D)) * ps[..., None]
    pm[0, [1, 4]] = -np.inf; ps[0, [1, 4]] = 0; po[0, [1, 4]] = 0     # empty segments
    pm[2] = -np.inf; ps[2] = 0; po[2] = 0                             # a row with no keys
    pm[3, 5] = 80.0                                                   # one dominant segment
    pm, ps, po = (a.astype(np.float32) for a in (pm, ps, po))
    for dt in (torch.float32, torch.bfloat16):
        o, lse = rf.segment_merge(dev_f32(pm), dev_f32(ps), dev_f32(po), dt)
        torch.cuda.synchronize()
        ro, rl = oracle.merge_partials(pm, ps, po)
        tol = (1e-5, 1e-5) if dt == torch.float32 else (ATOL, RTOL)
        assert_close(host(o), ro, *tol, "O")
        assert_close(host(lse), rl, 1e-5, 1e-6, "lse")
        assert np.all(host(o)[2] == 0) and np.isneginf(host(lse)[2])


def test_many_segments_merge(rf):
    g = np.random.default_rng(6)
    R, T, D = 5, 1000, 64
    pm = (g.standard_normal((R, T)) * 3).astype(np.float32)
    ps = g.uniform(0.5, 30, (R, T)).astype(np.float32)
    po = (g.standard_normal((R, T, D)) * ps[..., None]).astype(np.float32)
    o, lse = rf.segment_merge(dev_f32(pm), dev_f32(ps), dev_f32(po), torch.float32)
    torch.cuda.synchronize()
    ro, rl = oracle.merge_partials(pm, ps, po)
    assert_close(host(o), ro, 1e-5, 1e-5, "O")
    assert_close(host(lse), rl, 1e-5, 1e-6, "lse")


def test_deterministic(rf):
    a = _check_case(rf, 1, 2, 300, 128, 4, seed=12)
    b = _check_case(rf, 1, 2, 300, 128, 4, seed=12)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("B,H,L,D", [
    (2, 4, 300, 128),     # 8 rows: two 150-key segments
    (1, 1, 5000, 64),     # one row: 39 segments of 129 keys
    (2, 2, 70, 128),      # shorter than one 128-key segment
    (8, 32, 2048, 128),   # 256 rows: four segments
])
def test_automatic_segment_count(rf, B, H, L, D):
    """rf_attn_decode_segments' choice goes through the same split + merge."""
    nseg = rf.attn_decode_segments(B * H, L)
    assert 1 <= nseg <= min(L, 1024)
    _check_case(rf, B, H, L, D, nseg, seed=40 + L)


@pytest.mark.slow
@pytest.mark.parametrize("nseg", [8, 32, None])
def test_decode_l2048_full(rf, nseg):
    """The L = 2048 workload (32 x 32 heads, D = 128) checked on every head."""
    c = CONFIGS["C3a"]
    B, H, L, D = c["B"], c["H"], c["L"], c["D"]
    q, k, v, scale = decode_inputs(B, H, L, D, c["seed"])
    o, lse = rf.attn_decode(dev_bf16(q), dev_bf16(k), dev_bf16(v), nseg, scale)
    torch.cuda.synchronize()
    go, gl = host(o), host(lse)
    qf = _f(q)
    for b0 in range(0, B, 8):      # oracle in chunks of 8 batches to bound host memory
        ro, rl = oracle.decode(qf[b0:b0 + 8], _f(k[b0:b0 + 8]), _f(v[b0:b0 + 8]), scale)
        assert_close(go[b0:b0 + 8], ro, ATOL, RTOL, f"O batches {b0}..")
        assert_close(gl[b0:b0 + 8], rl, ATOL, RTOL, f"lse batches {b0}..")


@pytest.mark.slow
@pytest.mark.parametrize("nseg", [32, None])
def test_decode_l16384_sampled(rf, nseg):
    """The L = 16384 workload (8 GiB of K/V): every head computed, 24 heads checked
    against the oracle regenerated slice by slice; 64-bit offsets are exercised."""
    c = CONFIGS["C3b"]
    B, H, L, D = c["B"], c["H"], c["L"], c["D"]
    q, k, v, scale = decode_inputs(B, H, L, D, c["seed"])
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    del k, v
    o, lse = rf.attn_decode(dq, dk, dv, nseg, scale)
    torch.cuda.synchronize()
    go, gl = host(o), host(lse)
    g = np.random.default_rng(7)
    heads = [(0, 0), (B - 1, H - 1), (B - 1, 0)] + [tuple(x) for x in g.integers(0, [B, H], (21, 2))]
    qd = decode_q(B, H, D, c["seed"])
    for (b, h), ro, rl in oracle.decode_streaming(
            lambda b, h: _f(qd[b, h]), lambda b, h: tuple(_f(t) for t in decode_kv_slice(b, h, L, D, c["seed"])),
            heads, scale):
        assert_close(go[b, h], ro, ATOL, RTOL, f"O[{b},{h}]")
        assert_close(gl[b, h], rl, ATOL, RTOL, f"lse[{b},{h}]")


@pytest.mark.parametrize("B,H,L,D,nseg", [
    (2, 4, 300, 128, 1),      # one segment: a single launch writes o and lse
    (1, 3, 1, 64, 1),         # one key
    (2, 2, 517, 64, 1),
    (2, 4, 300, 128, 3),      # split + merge through the workspace
    (4, 8, 1000, 128, 0),     # automatic count
])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_one_call_decode(rf, B, H, L, D, nseg, out_dtype):
    q, k, v, scale = decode_inputs(B, H, L, D, seed=70 + L + nseg)
    o, lse = rf.attn_decode(dev_bf16(q), dev_bf16(k), dev_bf16(v), nseg or None, scale, out_dtype)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(_f(q), _f(k), _f(v), scale)
    atol, rtol = (ATOL, RTOL) if out_dtype == torch.bfloat16 else (1e-3, 1e-3)
    assert_close(host(o), ro, atol, rtol, "O")
    assert_close(host(lse), rl, ATOL, RTOL, "lse")


_RNG_SHAPES = np.random.default_rng(1024)
RANDOM = [(int(_RNG_SHAPES.integers(1, 4)), int(_RNG_SHAPES.integers(1, 9)), int(_RNG_SHAPES.integers(1, 3000)),
           int(_RNG_SHAPES.choice([64, 128])), int(_RNG_SHAPES.integers(1, 40))) for _ in range(8)]


@pytest.mark.parametrize("B,H,L,D,nseg", RANDOM)
def test_random_shapes(rf, B, H, L, D, nseg):
    """Seeded random shapes and segment counts (including more segments than keys)."""
    _check_case(rf, B, H, L, D, nseg, seed=1300 + L + nseg)
