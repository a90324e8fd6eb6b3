"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and bench.py.

This module draws random numbers and packs them into the storage formats the
library reads (fp32, bf16 bit patterns, e4m3fn codes). It holds none of the
fused method's arithmetic: no scores, maxima, sums, top-k or quantisation of
activations happen here. The two pieces of arithmetic it does contain are input
conditioning, each documented where it sits:

* ``moe_inputs`` re-draws tokens whose top expert scores nearly tie, so that the
  top-k selection is unique and robust to fp32 accumulation order;
* ``quant_inputs`` stores the weight already quantised per column (the weight is
  an input in pre-quantised form, not a step of the method), using torch's own
  fp8 cast as a library routine.

Every generator is a pure function of (seed, shape): numpy
``Generator(PCG64(SeedSequence([seed, *keys])))`` with fp32 standard normals,
tensors drawn in the order listed in each docstring. bf16 values are produced
by round-to-nearest-even on the fp32 bit pattern, so the oracle and the GPU see
identical bytes.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os as _os
from dataclasses import dataclass

import numpy as np

__all__ = [
    "rng", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "attn_inputs", "decode_q", "decode_kv_slice", "decode_inputs",
    "moe_inputs", "quant_inputs", "CONFIGS",
]


def rng(seed: int, *keys: int) -> np.random.Generator:
    """A PCG64 stream keyed by (seed, *keys)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), *map(int, keys)])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest, ties to even. Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the exactly equal fp32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_f32(g: np.random.Generator, shape) -> np.ndarray:
    return g.standard_normal(size=shape, dtype=np.float32)


# ---------------------------------------------------------------- attention (prefill)

@dataclass
class AttnInputs:
    q: np.ndarray  # fp32 [B,H,Sq,D] or bf16 bits uint16
    k: np.ndarray
    v: np.ndarray
    scale: float   # the fp32 softmax scale as passed to the library
    dtype: str     # "f32" | "bf16"


def attn_inputs(B: int, H: int, Sq: int, Sk: int, D: int, dtype: str, seed: int,
                scale: float | None = None) -> AttnInputs:
    """Q, K, V i.i.d. N(0,1), drawn in the order Q, K, V from rng(seed).

    dtype "f32" keeps fp32 values; "bf16" returns RNE bf16 bit patterns.
    The default scale is fl32(1/sqrt(D)).
    """
    g = rng(seed)
    q = _normal_f32(g, (B, H, Sq, D))
    k = _normal_f32(g, (B, H, Sk, D))
    v = _normal_f32(g, (B, H, Sk, D))
    if scale is None:
        scale = float(np.float32(1.0 / np.sqrt(D)))
    if dtype == "bf16":
        q, k, v = f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)
    elif dtype != "f32":
        raise ValueError(dtype)
    return AttnInputs(q, k, v, float(np.float32(scale)), dtype)


# ---------------------------------------------------------------- decode (one query token)

def decode_q(B: int, H: int, D: int, seed: int) -> np.ndarray:
    """q [B,H,D] bf16 bits from rng(seed, 0)."""
    return f32_to_bf16_bits(_normal_f32(rng(seed, 0), (B, H, D)))


def decode_kv_slice(b: int, h: int, L: int, D: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """K[b,h] and V[b,h] ([L,D] bf16 bits), each from its own child stream
    rng(seed, 1, b, h, tensor_id) so any head can be regenerated alone."""
    k = f32_to_bf16_bits(_normal_f32(rng(seed, 1, b, h, 0), (L, D)))
    v = f32_to_bf16_bits(_normal_f32(rng(seed, 1, b, h, 1), (L, D)))
    return k, v


def decode_inputs(B: int, H: int, L: int, D: int, seed: int, threads: int | None = None):
    """Full decode inputs: q [B,H,D], K and V [B,H,L,D] (bf16 bits), scale fl32(1/sqrt(D)).

    Heads are generated in parallel threads (numpy releases the GIL while
    filling); the result is independent of the thread count."""
    q = decode_q(B, H, D, seed)
    k = np.empty((B, H, L, D), np.uint16)
    v = np.empty((B, H, L, D), np.uint16)

    def fill(bh):
        b, h = divmod(bh, H)
        k[b, h], v[b, h] = decode_kv_slice(b, h, L, D, seed)

    n = threads or min(16, _os.cpu_count() or 1)
    with _cf.ThreadPoolExecutor(n) as ex:
        list(ex.map(fill, range(B * H)))
    return q, k, v, float(np.float32(1.0 / np.sqrt(D)))


# ---------------------------------------------------------------- MLA decode (latent cache)

MLA_DQK, MLA_DV, MLA_QK_HEAD = 576, 512, 192


def mla_q(B: int, H: int, seed: int) -> np.ndarray:
    """Absorbed queries q [B,H,576] bf16 bits from rng(seed, 0)."""
    return f32_to_bf16_bits(_normal_f32(rng(seed, 0), (B, H, MLA_DQK)))


def mla_kv_slice(b: int, L: int, seed: int) -> np.ndarray:
    """Cache rows kv[b] [L,576] bf16 bits (latent 512 then rotary 64) from rng(seed, 1, b)."""
    return f32_to_bf16_bits(_normal_f32(rng(seed, 1, b), (L, MLA_DQK)))


def mla_inputs(B: int, H: int, L: int, seed: int):
    """q [B,H,576], kv [B,L,576] (bf16 bits) and the scale fl32(1/sqrt(192)) (the softmax
    scale of a 128 + 64 query-key head, whose product the absorbed form preserves)."""
    q = mla_q(B, H, seed)
    kv = np.empty((B, L, MLA_DQK), np.uint16)

    def fill(b):
        kv[b] = mla_kv_slice(b, L, seed)

    with _cf.ThreadPoolExecutor(min(16, _os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(B)))
    return q, kv, float(np.float32(1.0 / np.sqrt(MLA_QK_HEAD)))


# ---------------------------------------------------------------- MoE gate

def _near_tie_rows(x_bits: np.ndarray, w_bits: np.ndarray, k: int, gap: float) -> np.ndarray:
    """Rows whose k+1 largest fp64 gate scores have a neighbouring gap < `gap`.

    Input conditioning only: it decides which tokens to draw again so that the
    top-k set and its order are unique and far from fp32 rounding noise."""
    s = bf16_bits_to_f32(x_bits).astype(np.float64) @ bf16_bits_to_f32(w_bits).astype(np.float64)
    top = -np.sort(-s, axis=1)[:, : min(k + 1, s.shape[1])]
    gaps = top[:, :-1] - top[:, 1:]
    return np.nonzero((gaps < gap).any(axis=1))[0]


def moe_inputs(T: int, Hd: int, E: int, k: int, seed: int, gap: float = 1e-2, w_std: float = 0.02):
    """X [T,Hd] ~ N(0,1) and W_gate [Hd,E] ~ N(0, w_std^2), both bf16 bits.

    Drawn in the order W_gate, then X (row by row from one stream). Each token
    whose (j, j+1)-th largest score gap, for j = 1..k, is below `gap` is
    re-drawn from the same stream, in row order, until none remain. With
    gap <= 0 no token is re-drawn.
    """
    g = rng(seed)
    w = f32_to_bf16_bits(_normal_f32(g, (Hd, E)) * np.float32(w_std))
    x = f32_to_bf16_bits(_normal_f32(g, (T, Hd)))
    if gap > 0 and E > k:
        for _ in range(10_000):
            bad = _near_tie_rows(x, w, k, gap)
            if bad.size == 0:
                break
            for r in bad:
                x[r] = f32_to_bf16_bits(_normal_f32(g, (Hd,)))
        else:  # pragma: no cover
            raise RuntimeError("rejection sampling did not converge")
    return x, w


# ---------------------------------------------------------------- FP8 quant GEMM

def quant_inputs(M: int, N: int, K: int, seed: int, outlier_p: float = 0.01, outlier_mul: float = 20.0):
    """Activations X and a pre-quantised weight.

    Drawn in the order X (N(0,1) fp32), the outlier mask (Bernoulli(outlier_p)
    per element, those elements multiplied by outlier_mul before bf16
    rounding), then W_f [N,K] ~ N(0,1) fp32.

    Returns (x_bits [M,K] bf16, wq [N,K] uint8 e4m3fn codes, w_scale [N] fp32).
    Row j of wq holds column j of the logical K x N weight (K contiguous, the
    layout of a linear layer's weight). The weight is stored pre-quantised per
    column: w_scale[j] = fl32(max_k |W_f[j,k]| / 448) and wq = e4m3fn(fl32(W_f / w_scale)),
    the fp8 cast being torch's (round to nearest even).
    """
    import torch  # library fp8 cast, used only to pre-quantise the weight input

    g = rng(seed)
    x = _normal_f32(g, (M, K))
    mask = g.random(size=(M, K), dtype=np.float32) < np.float32(outlier_p)
    x = np.where(mask, x * np.float32(outlier_mul), x).astype(np.float32)
    x_bits = f32_to_bf16_bits(x)
    wf = _normal_f32(g, (N, K))
    amax = np.abs(wf).max(axis=1)
    w_scale = (amax / np.float32(448.0)).astype(np.float32)
    w_scale = np.where(w_scale == 0, np.float32(1.0), w_scale).astype(np.float32)
    ratio = (wf / w_scale[:, None]).astype(np.float32)
    wq = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    return x_bits, wq, w_scale


# ---------------------------------------------------------------- the five workloads

CONFIGS = {
    # name: (generator, kwargs)
    "C1": dict(kind="attn", B=1, H=1, Sq=64, Sk=256, D=64, dtype="f32", seed=1, scale=0.125),
    "C2": dict(kind="attn", B=8, H=12, Sq=512, Sk=512, D=64, dtype="bf16", seed=2, scale=0.125),
    "C3a": dict(kind="decode", B=32, H=32, L=2048, D=128, seed=3),
    "C3b": dict(kind="decode", B=32, H=32, L=16384, D=128, seed=4),
    "C4": dict(kind="moe", T=2048, Hd=4096, E=64, k=2, seed=5),
    "C5": dict(kind="quant", M=4096, N=4096, K=4096, seed=6),
    # Multi-head latent attention decode (a workload beyond the five above): 32 sequences,
    # 128 heads sharing a 576-wide latent cache of 4096 tokens.
    "MLA": dict(kind="mla", B=32, H=128, L=4096, seed=7),
}
