"""GPU parity: rf_mla_decode_split + rf_segment_merge (D = 512) against the oracle.

Merged outputs are compared with the plain definition (oracle.mla_decode). The
split partials carry a lazily moved reference, so they are compared through
quantities that do not depend on it: each segment's log-sum-exp
(part_m + ln part_s) and its normalised output (part_o / part_s)."""
import numpy as np
import pytest
import torch

import oracle
from synth import CONFIGS, bf16_bits_to_f32, mla_inputs, mla_kv_slice, mla_q
from tests.gpu_util import assert_close, dev_bf16, host

pytestmark = pytest.mark.gpu

ATOL, RTOL = 2e-2, 1e-2
DV = 512


def _f(bits):
    return bf16_bits_to_f32(bits).astype(np.float64)


def _check(rf, B, H, L, nseg, seed, scale=None):
    q, kv, sc = mla_inputs(B, H, L, seed)
    scale = sc if scale is None else scale
    dq, dkv = dev_bf16(q), dev_bf16(kv)
    pm, ps, po = rf.mla_decode_split(dq, dkv, nseg, scale)
    o, lse = rf.segment_merge(pm, ps, po, torch.bfloat16)
    torch.cuda.synchronize()
    qf, kvf = _f(q), _f(kv)
    ro, rl = oracle.mla_decode(qf, kvf, DV, scale)
    assert_close(host(o).reshape(B, H, DV), ro, ATOL, RTOL, "O")
    assert_close(host(lse).reshape(B, H), rl, ATOL, RTOL, "lse")
    # Per-segment checks through reference-free quantities.
    rpm, rps, rpo = oracle.split_partials(qf.reshape(B * H, -1), np.repeat(kvf, H, axis=0),
                                          np.repeat(kvf[..., :DV], H, axis=0), scale, nseg)
    gm, gs, go = host(pm), host(ps), host(po)
    nonempty = rps > 0
    assert np.array_equal(gs > 0, nonempty)
    seg_lse = np.where(nonempty, gm + np.log(np.where(gs > 0, gs, 1.0)), -np.inf)
    ref_lse = np.where(nonempty, rpm + np.log(np.where(nonempty, rps, 1.0)), -np.inf)
    assert_close(seg_lse, ref_lse, 5e-3, 1e-3, "segment lse")
    g_norm = go / np.where(gs > 0, gs, 1.0)[..., None]
    r_norm = rpo / np.where(nonempty, rps, 1.0)[..., None]
    assert_close(g_norm, r_norm, ATOL, RTOL, "segment outputs")
    return host(o)


@pytest.mark.parametrize("B,H,L,nseg", [
    (1, 64, 100, 1),       # one segment, ragged last tile
    (2, 32, 300, 3),       # H = 32: half of the workgroup's heads are past H
    (2, 128, 513, 4),      # two head blocks, a one-token tail
    (1, 64, 31, 1),        # a single partial tile
    (1, 96, 200, 7),       # H = 96
    (1, 64, 7, 5),         # segments of 2 tokens, the last one empty
    (2, 64, 1000, 16),
])
def test_mla_split_merge(rf, B, H, L, nseg):
    _check(rf, B, H, L, nseg, seed=50 + L + nseg)


@pytest.mark.parametrize("scale", [0.0, -0.0721688, 0.5])
def test_mla_scales(rf, scale):
    """Zero (every weight equal), negative and large scales (the reference must move)."""
    _check(rf, 1, 64, 257, 2, seed=61, scale=scale)


@pytest.mark.parametrize("growth,nseg", [(12.0, 1), (60.0, 1), (60.0, 3)])
def test_mla_growing_scores(rf, growth, nseg):
    """Cache rows pushed along the heads' mean query direction, more for later tokens, so
    every head's scores grow along the sequence by about `growth` (natural units): the
    reference maximum moves again and again inside the software-pipelined tile loop."""
    from synth import f32_to_bf16_bits
    B, H, L = 1, 64, 640
    q, kv, scale = mla_inputs(B, H, L, 64)
    qf, kvf = _f(q), _f(kv)
    qm = qf.mean(axis=1)                                     # [B, 576]
    c = np.linspace(0.0, growth / (scale * (qm ** 2).sum()), L)
    kv = f32_to_bf16_bits((kvf + c[None, :, None] * qm[:, None, :]).astype(np.float32))
    dq, dkv = dev_bf16(q), dev_bf16(kv)
    pm, ps, po = rf.mla_decode_split(dq, dkv, nseg, scale)
    o, lse = rf.segment_merge(pm, ps, po, torch.bfloat16)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(qf, _f(kv), DV, scale)
    assert_close(host(o).reshape(B, H, DV), ro, ATOL, RTOL, "O")
    assert_close(host(lse).reshape(B, H), rl, ATOL, RTOL, "lse")


def test_mla_automatic_segments(rf):
    q, kv, scale = mla_inputs(4, 128, 640, 62)
    o, lse = rf.mla_decode(dev_bf16(q), dev_bf16(kv), scale)
    torch.cuda.synchronize()
    ro, rl = oracle.mla_decode(_f(q), _f(kv), DV, scale)
    assert_close(host(o), ro, ATOL, RTOL, "O")
    assert_close(host(lse), rl, ATOL, RTOL, "lse")


def test_mla_deterministic(rf):
    q, kv, scale = mla_inputs(2, 64, 400, 63)
    a = rf.mla_decode(dev_bf16(q), dev_bf16(kv), scale, nseg=3)[0]
    b = rf.mla_decode(dev_bf16(q), dev_bf16(kv), scale, nseg=3)[0]
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.slow
def test_mla_workload_sampled(rf):
    """The 32 x 128-head, 4096-token workload with the automatic segment count: every
    output computed, 6 batch entries (all heads) checked, regenerated entry by entry."""
    c = CONFIGS["MLA"]
    B, H, L = c["B"], c["H"], c["L"]
    q, kv, scale = mla_inputs(B, H, L, c["seed"])
    o, lse = rf.mla_decode(dev_bf16(q), dev_bf16(kv), scale)
    torch.cuda.synchronize()
    go, gl = host(o), host(lse)
    qd = mla_q(B, H, c["seed"])
    for b in (0, 1, 7, 16, 30, B - 1):
        ro, rl = oracle.mla_decode(_f(qd[b:b + 1]), _f(mla_kv_slice(b, L, c["seed"]))[None], DV, scale)
        assert_close(go[b], ro[0], ATOL, RTOL, f"O[{b}]")
        assert_close(gl[b], rl[0], ATOL, RTOL, f"lse[{b}]")
