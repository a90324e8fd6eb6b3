"""Python binding of librf (fused cascaded reductions on MI355X).

A thin ctypes layer over the C ABI in include/librf.h: it checks tensor dtype,
device, shape and contiguity, passes data pointers and the current HIP stream,
and turns a non-zero status into RFError. All arithmetic happens in the HIP
kernels; torch provides device memory and streams only. There is no fallback:
if librf.so is missing or cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

__all__ = [
    "RFError", "load", "lib_path", "RF_F32", "RF_BF16", "RF_ATTN_AUTO", "RF_ATTN_INCREMENTAL", "RF_ATTN_WHOLE_ROW",
    "softmax_gemm_fused", "attn_decode_split", "segment_merge", "attn_decode", "attn_decode_noalloc",
    "attn_decode_segments",
    "mla_decode_split", "mla_decode", "row_cascade", "cascade_gemm",
    "moe_route", "moe_route_split", "quant_gemm", "quant_gemm_workspace_size",
]

HERE = os.path.dirname(os.path.abspath(__file__))
ABI_VERSION = 5
RF_F32, RF_BF16 = 0, 1
_STATUS = {0: "RF_OK", 1: "RF_ERR_INVALID_ARGUMENT", 2: "RF_ERR_UNSUPPORTED",
           3: "RF_ERR_BUFFER_TOO_SMALL", 4: "RF_ERR_DEVICE"}


class RFError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{_STATUS.get(status, status)}: {message}")


def lib_path() -> str:
    return os.path.join(HERE, "librf.so")


_lib = None
_c = ctypes
_P, _I64, _F, _SZ = _c.c_void_p, _c.c_int64, _c.c_float, _c.c_size_t
_SIGS = {
    "rf_abi_version": ([], _c.c_int),
    "rf_status_string": ([_c.c_int], _c.c_char_p),
    "rf_last_error": ([], _c.c_char_p),
    "rf_softmax_gemm_fused": ([_c.c_int, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _P], _c.c_int),
    "rf_softmax_gemm_fused_mode": ([_c.c_int, _c.c_int, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _P],
                                   _c.c_int),
    "rf_attn_decode_split": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _P, _P, _P, _P], _c.c_int),
    "rf_segment_merge": ([_P, _P, _P, _I64, _I64, _I64, _c.c_int, _P, _P, _P], _c.c_int),
    "rf_attn_decode_segments": ([_I64, _I64, _I64], _I64),
    "rf_attn_decode_workspace_size": ([_I64, _I64, _I64, _I64, _I64], _SZ),
    "rf_attn_decode": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _c.c_int, _P, _P, _P, _SZ, _P], _c.c_int),
    "rf_attn_decode_noalloc": ([_P, _P, _P, _I64, _I64, _I64, _I64, _I64, _F, _c.c_int, _P, _P, _P], _c.c_int),
    "rf_mla_decode_split": ([_P, _P, _I64, _I64, _I64, _I64, _I64, _I64, _F, _P, _P, _P, _P], _c.c_int),
    "rf_row_cascade": ([_c.c_int, _P, _P, _I64, _I64, _I64, _I64, _P, _P, _P], _c.c_int),
    "rf_cascade_gemm": ([_c.c_int, _P, _P, _I64, _I64, _I64, _P, _P, _P], _c.c_int),
    "rf_moe_route": ([_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P], _c.c_int),
    "rf_moe_route_split_workspace_size": ([_I64, _I64, _I64], _SZ),
    "rf_moe_route_split": ([_P, _P, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P], _c.c_int),
    "rf_quant_gemm_workspace_size": ([_I64, _I64, _I64], _SZ),
    "rf_quant_gemm": ([_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P], _c.c_int),
    "rf_quant_gemm_fused": ([_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P], _c.c_int),
}


def load():
    """Load librf.so (once) and declare every exported signature. Raises RFError if absent."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RFError(-1, f"{path} is not built (python -m cascaded_reductions_amd.build)")
        lib = ctypes.CDLL(path)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes, fn.restype = args, res
        if lib.rf_abi_version() != ABI_VERSION:
            raise RFError(-1, f"unexpected ABI version {lib.rf_abi_version()}")
        _lib = lib
    return _lib


def _check(status: int):
    if status != 0:
        raise RFError(status, load().rf_last_error().decode())


def _torch():
    import torch
    return torch


def _need(t, name, dtype, shape=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    return t


def _ptr(t):
    return None if t is None else _c.c_void_p(t.data_ptr())


def _stream(t):
    return _c.c_void_p(_torch().cuda.current_stream(t.device).cuda_stream)


# ------------------------------------------------------------------ attention


RF_ATTN_AUTO, RF_ATTN_INCREMENTAL, RF_ATTN_WHOLE_ROW = 0, 1, 2
_MODES = {"auto": RF_ATTN_AUTO, "incremental": RF_ATTN_INCREMENTAL, "whole_row": RF_ATTN_WHOLE_ROW}


def softmax_gemm_fused(q, k, v, scale: float | None = None, *, out=None, lse=None, return_lse: bool = True,
                       mode: str = "auto"):
    """O = softmax(scale * Q K^T) V for q [B,H,Sq,D], k/v [B,H,Sk,D] (fp32 or bf16).

    mode: "auto" (whole-row below 256 keys for bf16, else incremental), "incremental" or
    "whole_row" (bf16, Sk <= 256). Returns (o, lse) with lse [B,H,Sq] fp32 (None if
    return_lse is False and no lse is given)."""
    if mode not in _MODES:
        raise ValueError(f"mode must be one of {sorted(_MODES)}")
    torch = _torch()
    dt = q.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    if q.dim() != 4:
        raise ValueError("q must be [B, H, Sq, D]")
    B, H, Sq, D = q.shape
    Sk = k.shape[2] if k.dim() == 4 else -1
    _need(q, "q", dt)
    _need(k, "k", dt, (B, H, Sk, D))
    _need(v, "v", dt, (B, H, Sk, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dt, q.shape)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (B, H, Sq))
    _check(load().rf_softmax_gemm_fused_mode(_MODES[mode], RF_F32 if dt == torch.float32 else RF_BF16, _ptr(q),
                                             _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, Sq, Sk, D, float(scale),
                                             _stream(q)))
    return out, lse


def attn_decode_split(q, k, v, nseg: int, scale: float | None = None, *, part_m=None, part_s=None, part_o=None):
    """Per-segment partials for q [B,H,D], k/v [B,H,L,D] bf16. Returns (part_m, part_s, part_o)."""
    torch = _torch()
    B, H, D = q.shape
    L = k.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, H, L, D))
    _need(v, "v", torch.bfloat16, (B, H, L, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dev = q.device
    part_m = torch.empty((B * H, nseg), dtype=torch.float32, device=dev) if part_m is None else part_m
    part_s = torch.empty((B * H, nseg), dtype=torch.float32, device=dev) if part_s is None else part_s
    part_o = torch.empty((B * H, nseg, D), dtype=torch.float32, device=dev) if part_o is None else part_o
    _need(part_m, "part_m", torch.float32, (B * H, nseg))
    _need(part_s, "part_s", torch.float32, (B * H, nseg))
    _need(part_o, "part_o", torch.float32, (B * H, nseg, D))
    _check(load().rf_attn_decode_split(_ptr(q), _ptr(k), _ptr(v), B, H, L, D, nseg, float(scale),
                                       _ptr(part_m), _ptr(part_s), _ptr(part_o), _stream(q)))
    return part_m, part_s, part_o


def segment_merge(part_m, part_s, part_o, out_dtype=None, *, out=None, lse=None, return_lse: bool = True):
    """Merge partials [R,T], [R,T], [R,T,D] -> (o [R,D] in out_dtype, lse [R])."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    R, T, D = part_o.shape
    _need(part_m, "part_m", torch.float32, (R, T))
    _need(part_s, "part_s", torch.float32, (R, T))
    _need(part_o, "part_o", torch.float32, (R, T, D))
    out = torch.empty((R, D), dtype=out_dtype, device=part_o.device) if out is None else out
    _need(out, "out", out_dtype, (R, D))
    if lse is None and return_lse:
        lse = torch.empty((R,), dtype=torch.float32, device=part_o.device)
    if lse is not None:
        _need(lse, "lse", torch.float32, (R,))
    _check(load().rf_segment_merge(_ptr(part_m), _ptr(part_s), _ptr(part_o), R, T, D,
                                   RF_F32 if out_dtype == torch.float32 else RF_BF16, _ptr(out), _ptr(lse),
                                   _stream(part_o)))
    return out, lse


def attn_decode_segments(rows: int, L: int, num_cus: int = 0) -> int:
    """The library's segment count for rows = B*H decode rows over L keys (rf_attn_decode_segments);
    num_cus <= 0 asks the current device."""
    n = int(load().rf_attn_decode_segments(int(rows), int(L), int(num_cus)))
    if n <= 0:
        raise RFError(1, load().rf_last_error().decode())
    return n


_ws_cache = {}


def _workspace(tag, device, nbytes):
    """A scratch buffer per (entry point, device, current stream), grown on demand. Calls on
    one stream are ordered, so they can share it; another stream gets its own buffer."""
    torch = _torch()
    key = (tag, device.type, device.index, torch.cuda.current_stream(device).cuda_stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def attn_decode(q, k, v, nseg: int | None = None, scale: float | None = None, out_dtype=None, *, out=None,
                lse=None):
    """Decode attention in one call (rf_attn_decode): returns (o [B,H,D], lse [B,H]). nseg None
    lets the library choose (one segment, a single launch, whenever the rows fill the chip)."""
    torch = _torch()
    B, H, D = q.shape
    L = k.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, H, L, D))
    _need(v, "v", torch.bfloat16, (B, H, L, D))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out_dtype = out_dtype or torch.bfloat16
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out_dtype must be float32 or bfloat16")
    n = 0 if nseg is None else int(nseg)
    out = torch.empty((B, H, D), dtype=out_dtype, device=q.device) if out is None else out
    _need(out, "out", out_dtype, (B, H, D))
    lse = torch.empty((B, H), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(lse, "lse", torch.float32, (B, H))
    need = int(load().rf_attn_decode_workspace_size(B, H, L, D, n))
    ws = _workspace("decode", q.device, need) if need else None
    _check(load().rf_attn_decode(_ptr(q), _ptr(k), _ptr(v), B, H, L, D, n, float(scale),
                                 RF_F32 if out_dtype == torch.float32 else RF_BF16, _ptr(out), _ptr(lse), _ptr(ws),
                                 need, _stream(q)))
    return out, lse


def attn_decode_noalloc(q, k, v, out, lse, nseg: int | None = None, scale: float | None = None):
    """rf_attn_decode_noalloc: decode attention with the partials in the library's static
    device scratch (no workspace and no allocation in the call; the caller passes out
    [B,H,D] bf16 or fp32 and lse [B,H] fp32). Concurrent calls on one GPU race on the scratch."""
    torch = _torch()
    B, H, D = q.shape
    L = k.shape[2]
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, H, L, D))
    _need(v, "v", torch.bfloat16, (B, H, L, D))
    if out.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("out must be float32 or bfloat16")
    _need(out, "out", out.dtype, (B, H, D))
    _need(lse, "lse", torch.float32, (B, H))
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    _check(load().rf_attn_decode_noalloc(_ptr(q), _ptr(k), _ptr(v), B, H, L, D, 0 if nseg is None else int(nseg),
                                         float(scale), RF_F32 if out.dtype == torch.float32 else RF_BF16, _ptr(out),
                                         _ptr(lse), _stream(q)))
    return out, lse


# ------------------------------------------------------------------ MLA decode

MLA_DQK, MLA_DV = 576, 512


def mla_decode_split(q, kv, nseg: int, scale: float, *, part_m=None, part_s=None, part_o=None):
    """Per-segment partials of MLA decode for q [B,H,576], kv [B,L,576] bf16 (value = the first
    512 entries of each row). Returns (part_m [B*H,nseg], part_s [B*H,nseg], part_o [B*H,nseg,512])."""
    torch = _torch()
    B, H, Dq = q.shape
    L = kv.shape[1]
    _need(q, "q", torch.bfloat16, (B, H, MLA_DQK))
    _need(kv, "kv", torch.bfloat16, (B, L, MLA_DQK))
    dev = q.device
    part_m = torch.empty((B * H, nseg), dtype=torch.float32, device=dev) if part_m is None else part_m
    part_s = torch.empty((B * H, nseg), dtype=torch.float32, device=dev) if part_s is None else part_s
    part_o = torch.empty((B * H, nseg, MLA_DV), dtype=torch.float32, device=dev) if part_o is None else part_o
    _need(part_m, "part_m", torch.float32, (B * H, nseg))
    _need(part_s, "part_s", torch.float32, (B * H, nseg))
    _need(part_o, "part_o", torch.float32, (B * H, nseg, MLA_DV))
    _check(load().rf_mla_decode_split(_ptr(q), _ptr(kv), B, H, L, MLA_DQK, MLA_DV, nseg, float(scale),
                                      _ptr(part_m), _ptr(part_s), _ptr(part_o), _stream(q)))
    return part_m, part_s, part_o


def mla_decode(q, kv, scale: float, nseg: int | None = None, out_dtype=None):
    """Split + merge: returns (o [B,H,512], lse [B,H]). With nseg None, the segment rule of
    attn_decode_segments counts the split kernel's waves (four per 64 heads)."""
    B, H, _ = q.shape
    if nseg is None:
        nseg = attn_decode_segments(max(1, B * H // 16), kv.shape[1])
    pm, ps, po = mla_decode_split(q, kv, nseg, scale)
    o, lse = segment_merge(pm, ps, po, out_dtype)
    return o.view(B, H, MLA_DV), lse.view(B, H)


# ------------------------------------------------------------------ generic row cascades

_CASCADES = {"logsumexp": 0, "softmax_weighted": 1, "topk_softmax": 2, "mean_var": 3}


def row_cascade(kind: str, x, payload=None, k: int = 0):
    """One of the library's template cascades over each row of x [R, N] fp32:
    "logsumexp" -> [R]; "softmax_weighted" (payload [R, N, P]) -> [R, P];
    "topk_softmax" -> (weights [R, k], indices [R, k] int32); "mean_var" -> [R, 2]."""
    torch = _torch()
    if kind not in _CASCADES:
        raise ValueError(f"kind must be one of {sorted(_CASCADES)}")
    R, N = x.shape
    _need(x, "x", torch.float32, (R, N))
    P = 0
    if kind == "softmax_weighted":
        P = payload.shape[2]
        _need(payload, "payload", torch.float32, (R, N, P))
    width = {"logsumexp": None, "softmax_weighted": P, "topk_softmax": k, "mean_var": 2}[kind]
    out = torch.empty((R,) if width is None else (R, width), dtype=torch.float32, device=x.device)
    idx = torch.empty((R, k), dtype=torch.int32, device=x.device) if kind == "topk_softmax" else None
    _check(load().rf_row_cascade(_CASCADES[kind], _ptr(x), _ptr(payload) if P else None, R, N, P, k, _ptr(out),
                                 _ptr(idx), _stream(x)))
    return (out, idx) if idx is not None else out


_CASCADE_GEMMS = {"softmax": 0, "absmax": 1}


def cascade_gemm(kind: str, x, w, *, y=None, stat=None):
    """A row-scaled GEMM cascade from the template: x [M, K] fp32, w [K, N] bf16 ->
    (y [M, N] fp32, stat [M] fp32). kind "softmax": y = softmax(x) w, stat = logsumexp(x);
    "absmax": y = (x / max|x|) w, stat = max|x|."""
    torch = _torch()
    if kind not in _CASCADE_GEMMS:
        raise ValueError(f"kind must be one of {sorted(_CASCADE_GEMMS)}")
    M, K = x.shape
    N = w.shape[1]
    _need(x, "x", torch.float32, (M, K))
    _need(w, "w", torch.bfloat16, (K, N))
    y = torch.empty((M, N), dtype=torch.float32, device=x.device) if y is None else y
    stat = torch.empty((M,), dtype=torch.float32, device=x.device) if stat is None else stat
    _need(y, "y", torch.float32, (M, N))
    _need(stat, "stat", torch.float32, (M,))
    _check(load().rf_cascade_gemm(_CASCADE_GEMMS[kind], _ptr(x), _ptr(w), M, K, N, _ptr(y), _ptr(stat), _stream(x)))
    return y, stat


# ------------------------------------------------------------------ MoE gate


def moe_route(x, w_gate, k: int, *, idx=None, w=None, scores=None, return_scores: bool = False):
    """x [T,Hd] bf16, w_gate [Hd,E] bf16 -> (idx [T,k] int32, w [T,k] fp32, scores [T,E] fp32 or None)."""
    torch = _torch()
    T, Hd = x.shape
    E = w_gate.shape[1]
    _need(x, "x", torch.bfloat16)
    _need(w_gate, "w_gate", torch.bfloat16, (Hd, E))
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if idx is None else idx
    w = torch.empty((T, k), dtype=torch.float32, device=x.device) if w is None else w
    _need(idx, "idx", torch.int32, (T, k))
    _need(w, "w", torch.float32, (T, k))
    if scores is None and return_scores:
        scores = torch.empty((T, E), dtype=torch.float32, device=x.device)
    if scores is not None:
        _need(scores, "scores", torch.float32, (T, E))
    _check(load().rf_moe_route(_ptr(x), _ptr(w_gate), T, Hd, E, k, _ptr(idx), _ptr(w), _ptr(scores), _stream(x)))
    return idx, w, scores


def moe_route_split(x, w_gate, k: int, *, idx=None, w=None, scores=None, return_scores: bool = False):
    """rf_moe_route_split: the two-launch form over a split hidden axis (scratch cached per
    device and stream). Same arguments and results as moe_route."""
    torch = _torch()
    T, Hd = x.shape
    E = w_gate.shape[1]
    _need(x, "x", torch.bfloat16)
    _need(w_gate, "w_gate", torch.bfloat16, (Hd, E))
    idx = torch.empty((T, k), dtype=torch.int32, device=x.device) if idx is None else idx
    w = torch.empty((T, k), dtype=torch.float32, device=x.device) if w is None else w
    _need(idx, "idx", torch.int32, (T, k))
    _need(w, "w", torch.float32, (T, k))
    if scores is None and return_scores:
        scores = torch.empty((T, E), dtype=torch.float32, device=x.device)
    if scores is not None:
        _need(scores, "scores", torch.float32, (T, E))
    need = int(load().rf_moe_route_split_workspace_size(T, Hd, E))
    ws = _workspace("moe_split", x.device, need)
    _check(load().rf_moe_route_split(_ptr(x), _ptr(w_gate), T, Hd, E, k, _ptr(idx), _ptr(w), _ptr(scores), _ptr(ws),
                                     ws.numel(), _stream(x)))
    return idx, w, scores


# ------------------------------------------------------------------ dynamic FP8 quant GEMM


def quant_gemm_workspace_size(M: int, N: int, K: int) -> int:
    return int(load().rf_quant_gemm_workspace_size(M, N, K))


def quant_gemm(x, wq, w_scale, *, y=None, x_scale=None, xq=None, workspace=None, return_codes: bool = False):
    """x [M,K] bf16, wq [N,K] uint8 (E4M3FN codes), w_scale [N] fp32 -> (y [M,N] bf16, x_scale [M], xq or None)."""
    torch = _torch()
    M, K = x.shape
    N = wq.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(wq, "wq", torch.uint8, (N, K))
    _need(w_scale, "w_scale", torch.float32, (N,))
    dev = x.device
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    x_scale = torch.empty((M,), dtype=torch.float32, device=dev) if x_scale is None else x_scale
    _need(y, "y", torch.bfloat16, (M, N))
    _need(x_scale, "x_scale", torch.float32, (M,))
    if xq is None and return_codes:
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if xq is not None:
        _need(xq, "xq", torch.uint8, (M, K))
    ws_bytes = 0
    if xq is None:
        need = quant_gemm_workspace_size(M, N, K)
        if workspace is None and need:
            workspace = torch.empty((need,), dtype=torch.uint8, device=dev)
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load().rf_quant_gemm(_ptr(x), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(y), _ptr(x_scale), _ptr(xq),
                                _ptr(workspace), ws_bytes, _stream(x)))
    return y, x_scale, xq


def quant_gemm_fused(x, wq, w_scale, *, y=None, x_scale=None, xq=None, return_codes: bool = False):
    """The same cascade as quant_gemm in one launch, with no workspace (rf_quant_gemm_fused)."""
    torch = _torch()
    M, K = x.shape
    N = wq.shape[0]
    _need(x, "x", torch.bfloat16)
    _need(wq, "wq", torch.uint8, (N, K))
    _need(w_scale, "w_scale", torch.float32, (N,))
    dev = x.device
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if y is None else y
    x_scale = torch.empty((M,), dtype=torch.float32, device=dev) if x_scale is None else x_scale
    _need(y, "y", torch.bfloat16, (M, N))
    _need(x_scale, "x_scale", torch.float32, (M,))
    if xq is None and return_codes:
        xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    if xq is not None:
        _need(xq, "xq", torch.uint8, (M, K))
    _check(load().rf_quant_gemm_fused(_ptr(x), _ptr(wq), _ptr(w_scale), M, N, K, _ptr(y), _ptr(x_scale), _ptr(xq),
                                      _stream(x)))
    return y, x_scale, xq
