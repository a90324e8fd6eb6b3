"""The C-ABI library loads, exports every symbol include/librf.h declares, and
rejects invalid arguments on the host (no GPU needed: validation runs before
any HIP call, and no call here passes validation)."""
import ctypes
import os
import re

import pytest

import cascaded_reductions_amd as rf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "librf.h")

OK, INVALID, UNSUPPORTED, TOO_SMALL, DEVICE = 0, 1, 2, 3, 4
P = 0x100000  # a fake, 16-byte aligned device address; never dereferenced
P2, P3, P4, P5, P6 = (P * i for i in range(2, 7))


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^RF_API\s+[\w\s\*]+?\b(rf_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    return rf.load()


def test_header_declares_the_boundary():
    assert declared_symbols() == sorted([
        "rf_abi_version", "rf_status_string", "rf_last_error", "rf_softmax_gemm_fused", "rf_softmax_gemm_fused_mode",
        "rf_attn_decode_split", "rf_segment_merge", "rf_attn_decode_segments", "rf_mla_decode_split", "rf_row_cascade",
        "rf_cascade_gemm",
        "rf_attn_decode_workspace_size", "rf_attn_decode", "rf_attn_decode_noalloc",
        "rf_moe_route", "rf_moe_route_split_workspace_size", "rf_moe_route_split",
        "rf_quant_gemm_workspace_size", "rf_quant_gemm", "rf_quant_gemm_fused"])


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_status_strings(lib):
    assert lib.rf_abi_version() == 5
    for code, name in [(0, b"RF_OK"), (1, b"RF_ERR_INVALID_ARGUMENT"), (2, b"RF_ERR_UNSUPPORTED"),
                       (3, b"RF_ERR_BUFFER_TOO_SMALL"), (4, b"RF_ERR_DEVICE")]:
        assert lib.rf_status_string(code) == name
    assert lib.rf_status_string(99) == b"RF_STATUS_UNKNOWN"


def _attn(lib, dt=0, q=P, k=P2, v=P3, o=P4, lse=None, B=1, H=1, Sq=4, Sk=4, D=64, scale=0.125):
    return lib.rf_softmax_gemm_fused(dt, q, k, v, o, lse, B, H, Sq, Sk, D, scale, None)


def test_attention_validation(lib):
    assert _attn(lib, dt=7) == INVALID
    assert _attn(lib, q=None) == INVALID
    assert b"q must not be NULL" in lib.rf_last_error()
    assert _attn(lib, k=P2 + 8) == INVALID
    assert b"aligned" in lib.rf_last_error()
    assert _attn(lib, lse=P5 + 4) == INVALID
    assert _attn(lib, Sq=0) == INVALID
    assert _attn(lib, Sk=-1) == INVALID
    assert _attn(lib, D=0) == INVALID
    assert _attn(lib, D=96) == UNSUPPORTED
    assert _attn(lib, D=256) == UNSUPPORTED
    assert _attn(lib, scale=float("inf")) == INVALID
    assert _attn(lib, scale=float("nan")) == INVALID
    assert _attn(lib, o=P) == INVALID                       # output aliases q
    assert _attn(lib, lse=P4 + 64) == INVALID               # lse inside o
    assert _attn(lib, B=1 << 40, H=1 << 30) == UNSUPPORTED  # overflow guarded


def _split(lib, q=P, k=P2, v=P3, B=2, H=2, L=64, D=128, nseg=8, pm=P4, ps=P5, po=P6):
    return lib.rf_attn_decode_split(q, k, v, B, H, L, D, nseg, 0.088, pm, ps, po, None)


def test_decode_split_validation(lib):
    assert _split(lib, q=None) == INVALID
    assert _split(lib, pm=None) == INVALID
    assert _split(lib, nseg=0) == INVALID
    assert _split(lib, nseg=65) == INVALID
    assert b"nseg" in lib.rf_last_error()
    n = lib.rf_attn_decode_noalloc
    assert n(P, P2, P3, 2, 4, 300, 96, 3, 0.08, 1, P4, None, None) == UNSUPPORTED        # D 96
    assert n(P, P2, P3, 2, 4, 300, 128, 3, 0.08, 1, P, None, None) == INVALID           # o over q
    assert n(P, P2, P3, 1 << 22, 1, 1024, 64, 1024, 0.1, 1, P4, None, None) == UNSUPPORTED
    assert _split(lib, L=0) == INVALID
    assert _split(lib, D=80) == UNSUPPORTED
    assert _split(lib, pm=P5) == INVALID                    # part_m aliases part_s


def _merge(lib, pm=P, ps=P2, po=P3, rows=4, nseg=8, D=128, dt=1, o=P4, lse=None):
    return lib.rf_segment_merge(pm, ps, po, rows, nseg, D, dt, o, lse, None)


def test_merge_validation(lib):
    assert _merge(lib, po=None) == INVALID
    assert _merge(lib, dt=5) == INVALID
    assert _merge(lib, rows=0) == INVALID
    assert _merge(lib, nseg=0) == INVALID
    assert _merge(lib, nseg=2048) == UNSUPPORTED
    assert _merge(lib, D=32) == UNSUPPORTED
    assert _merge(lib, o=P3) == INVALID
    assert _merge(lib, lse=P4 + 16) == INVALID


def _moe(lib, x=P, w=P2, T=8, Hd=64, E=64, k=2, idx=P3, wt=P4, sc=None):
    return lib.rf_moe_route(x, w, T, Hd, E, k, idx, wt, sc, None)


def test_moe_validation(lib):
    assert _moe(lib, x=None) == INVALID
    assert _moe(lib, k=0) == INVALID
    assert _moe(lib, k=65) == INVALID
    assert _moe(lib, k=9) == UNSUPPORTED
    assert _moe(lib, Hd=48) == UNSUPPORTED
    assert _moe(lib, Hd=1 << 26) == UNSUPPORTED
    assert _moe(lib, E=40) == UNSUPPORTED
    assert _moe(lib, E=512) == UNSUPPORTED
    assert _moe(lib, T=0) == INVALID
    assert _moe(lib, idx=P4) == INVALID                     # idx aliases w
    assert _moe(lib, sc=P + 16) == INVALID                  # scores inside x
    s = lib.rf_moe_route_split
    need = lib.rf_moe_route_split_workspace_size(2048, 4096, 64)
    assert need == 32 * 8 * 64 * 64 * 4                    # 32 token blocks x 8 hidden ranges of partial scores
    assert s(P, P2, 8, 64, 64, 2, P3, P4, None, None, 1 << 20, None) == TOO_SMALL
    assert s(P, P2, 8, 64, 64, 2, P3, P4, None, P6, lib.rf_moe_route_split_workspace_size(8, 64, 64) - 1,
             None) == TOO_SMALL
    assert s(P, P2, 8, 64, 64, 2, P3, P4, None, P + 64, 1 << 20, None) == INVALID   # workspace inside x
    assert s(P, P2, 8, 48, 64, 2, P3, P4, None, P6, 1 << 20, None) == UNSUPPORTED   # Hd 48


def _qg(lib, x=P, wq=P2, ws=P3, M=16, N=16, K=256, y=P4, xs=P5, xq=P6, work=None, nbytes=0):
    return lib.rf_quant_gemm(x, wq, ws, M, N, K, y, xs, xq, work, nbytes, None)


def test_quant_gemm_validation(lib):
    assert lib.rf_quant_gemm_workspace_size(16, 16, 256) == 16 * 256
    assert lib.rf_quant_gemm_workspace_size(0, 16, 256) == 0
    assert _qg(lib, x=None) == INVALID
    assert _qg(lib, xs=None) == INVALID
    assert _qg(lib, K=100) == UNSUPPORTED
    assert _qg(lib, M=0) == INVALID
    assert _qg(lib, xq=None) == TOO_SMALL
    assert _qg(lib, xq=None, work=P6, nbytes=16 * 256 - 1) == TOO_SMALL
    assert _qg(lib, y=P) == INVALID
    assert _qg(lib, xq=P4 + 16) == INVALID


def _qgf(lib, x=P, wq=P2, ws=P3, M=16, N=16, K=256, y=P4, xs=P5, xq=P6):
    return lib.rf_quant_gemm_fused(x, wq, ws, M, N, K, y, xs, xq, None)


def test_quant_gemm_fused_validation(lib):
    assert _qgf(lib, x=None) == INVALID
    assert _qgf(lib, ws=None) == INVALID
    assert _qgf(lib, xs=None) == INVALID
    assert _qgf(lib, K=100) == UNSUPPORTED
    assert _qgf(lib, K=64) == UNSUPPORTED
    assert _qgf(lib, N=0) == INVALID
    assert _qgf(lib, y=P) == INVALID                        # y aliases x
    assert _qgf(lib, xq=P4 + 16) == INVALID                 # codes inside y
    assert _qgf(lib, xs=P6 + 8) == INVALID                  # x_scale inside the codes
    assert _qgf(lib, M=1 << 21, K=1 << 20) == UNSUPPORTED   # M*K beyond 2^40


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError, match="GPU tensor"):
        rf.softmax_gemm_fused(q, q, q)


def test_decode_segment_rule(lib):
    """One wave per SIMD (rows * nseg >= 4 * CUs) with the fewest segments, segments of at
    least 128 keys, at most 1024 segments."""
    seg = lib.rf_attn_decode_segments
    assert seg(1024, 2048, 256) == 1          # 32 x 32 heads already fill every SIMD
    assert seg(1024, 16384, 256) == 1
    assert seg(4096, 512, 256) == 1
    assert seg(256, 2048, 256) == 4           # 8 x 32 heads: 4 segments -> 1024 waves
    assert seg(32, 131072, 256) == 32
    assert seg(300, 4096, 256) == 4           # ceil(1024 / 300)
    assert seg(256, 256, 256) == 2            # capped by 128-key segments
    assert seg(1, 100, 256) == 1
    assert seg(1, 10 ** 6, 256) == 1024       # the merge's limit
    assert seg(8, 300, 304) == 2
    for rows in (1, 3, 64, 255, 1000):
        for L in (1, 127, 128, 5000, 70000):
            n = seg(rows, L, 256)
            assert 1 <= n <= min(L, 1024)
            assert n == 1 or L // n >= 128
            if n < min(1024, max(1, L // 128)):
                assert rows * n >= 1024 and rows * (n - 1) < 1024
    assert seg(0, 10, 256) == 0 and b"rows and L" in lib.rf_last_error()
    assert seg(5, 0, 256) == 0


def test_attention_mode_validation(lib):
    m = lib.rf_softmax_gemm_fused_mode
    args = (P, P2, P3, P4, None, 1, 1, 4, 4, 64, 0.125, None)
    assert m(3, 1, *args) == INVALID and b"mode" in lib.rf_last_error()
    assert m(2, 0, *args) == UNSUPPORTED and b"RF_ATTN_WHOLE_ROW" in lib.rf_last_error()   # fp32
    long_args = (P, P2, P3, P4, None, 1, 1, 4, 257, 64, 0.125, None)
    assert m(2, 1, *long_args) == UNSUPPORTED                                               # Sk > 256
    assert m(1, 1, P, None, P3, P4, None, 1, 1, 4, 4, 64, 0.125, None) == INVALID           # k NULL


def test_mla_validation(lib):
    m = lib.rf_mla_decode_split
    ok_args = dict(q=P, kv=P2, B=1, H=64, L=100, dqk=576, dv=512, nseg=2, scale=0.07, pm=P3, ps=P4, po=P5)

    def call(**kw):
        a = dict(ok_args, **kw)
        return m(a["q"], a["kv"], a["B"], a["H"], a["L"], a["dqk"], a["dv"], a["nseg"], a["scale"], a["pm"], a["ps"],
                 a["po"], None)
    assert call(q=None) == INVALID
    assert call(H=48) == UNSUPPORTED and b"multiple of 32" in lib.rf_last_error()
    assert call(dqk=512) == UNSUPPORTED
    assert call(nseg=101) == INVALID
    assert call(nseg=0) == INVALID
    assert call(L=0) == INVALID
    assert call(scale=float("nan")) == INVALID
    assert call(po=P) == INVALID and b"alias" in lib.rf_last_error()       # part_o over q
    assert lib.rf_segment_merge(P, P2, P3, 4, 2, 256, 1, P4, None, None) == UNSUPPORTED   # D 256


def test_row_cascade_validation(lib):
    c = lib.rf_row_cascade
    assert c(4, P, None, 2, 8, 0, 0, P2, None, None) == INVALID                 # unknown kind
    assert c(0, None, None, 2, 8, 0, 0, P2, None, None) == INVALID              # x NULL
    assert c(0, P, None, 0, 8, 0, 0, P2, None, None) == INVALID                 # R = 0
    assert c(1, P, None, 2, 8, 4, 0, P2, None, None) == INVALID                 # payload NULL
    assert c(1, P, P3, 2, 8, 3, 0, P2, None, None) == UNSUPPORTED               # P = 3
    assert c(0, P, None, 2, 8, 2, 0, P2, None, None) == INVALID                 # P for logsumexp
    assert c(2, P, None, 2, 8, 0, 9, P2, P3, None) == UNSUPPORTED               # k > 8
    assert c(2, P, None, 2, 4, 0, 5, P2, P3, None) == UNSUPPORTED               # k > N
    assert c(2, P, None, 2, 8, 0, 2, P2, None, None) == INVALID                 # out_idx NULL
    assert c(3, P, None, 2, 8, 0, 0, P, None, None) == INVALID                  # out over x


def test_decode_one_call_validation(lib):
    ws = lib.rf_attn_decode_workspace_size
    assert ws(32, 32, 2048, 128, 1) == 0                      # one segment: no partials
    assert ws(2, 4, 300, 128, 3) == 2 * 256 + (8 * 3 * 128 * 4 + 255) // 256 * 256
    assert ws(2, 4, 300, 96, 3) == 0 and ws(2, 4, 300, 128, 301) == 0
    d = lib.rf_attn_decode

    def call(nseg=3, ws_bytes=0, wsp=None, o=P4, D=128, L=300):
        return d(P, P2, P3, 2, 4, L, D, nseg, 0.08, 1, o, None, wsp, ws_bytes, None)
    assert call(ws_bytes=16) == TOO_SMALL and b"workspace" in lib.rf_last_error()
    assert call(nseg=301) == INVALID
    assert call(nseg=-1) == INVALID
    assert call(D=96) == UNSUPPORTED
    assert call(o=P) == INVALID                               # o over q
    need = ws(2, 4, 300, 128, 3)
    assert call(ws_bytes=need, wsp=P4) == INVALID             # workspace over o
    # 2^22 rows x 1024 segments: more split waves than the launch can index, refused on the host
    assert d(P, P2, P3, 1 << 22, 1, 1024, 64, 1024, 0.1, 1, P4, None, P5, 1 << 40, None) == UNSUPPORTED
    assert b"nseg" in lib.rf_last_error()
    n = lib.rf_attn_decode_noalloc
    assert n(P, P2, P3, 2, 4, 300, 96, 3, 0.08, 1, P4, None, None) == UNSUPPORTED        # D 96
    assert n(P, P2, P3, 2, 4, 300, 128, 3, 0.08, 1, P, None, None) == INVALID           # o over q
    assert n(P, P2, P3, 1 << 22, 1, 1024, 64, 1024, 0.1, 1, P4, None, None) == UNSUPPORTED


def test_cascade_gemm_validation(lib):
    c = lib.rf_cascade_gemm
    assert c(2, P, P2, 8, 64, 64, P3, None, None) == INVALID                    # unknown kind
    assert c(0, None, P2, 8, 64, 64, P3, None, None) == INVALID                 # x NULL
    assert c(0, P, P2, 0, 64, 64, P3, None, None) == INVALID                    # M = 0
    assert c(0, P, P2, 8, 64, 96, P3, None, None) == UNSUPPORTED                # N = 96
    assert c(1, P, P2, 8, 66, 64, P3, None, None) == UNSUPPORTED                # K % 4
    assert c(1, P, P2, 8, 1 << 24, 64, P3 * 1000, None, None) == UNSUPPORTED    # K too long
    assert c(0, P, P2, 8, 64, 64, P, None, None) == INVALID                     # y over x
    assert c(0, P, P2, 8, 64, 64, P3, P3 + 16, None) == INVALID                 # stat over y
    assert c(0, P + 8, P2, 8, 64, 64, P3, None, None) == INVALID                # misaligned x
