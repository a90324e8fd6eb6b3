"""GPU test of rf_attn_decode_noalloc (the decode call that allocates nothing: its segment
partials live in the library's static device scratch). Called through the C ABI and
compared with rf_attn_decode (caller workspace) on the same inputs: the two run the same
kernels in the same order, so the outputs must agree bit for bit. Two calls in a row, the
second smaller, so the scratch holds the first call's partials when the second starts."""
import ctypes

import numpy as np
import pytest
import torch

from synth import decode_inputs
from tests.gpu_util import dev_bf16

pytestmark = pytest.mark.gpu

RF_BF16, RF_F32 = 1, 0


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _run_both(lib, B, H, L, D, nseg, out_dtype, seed):
    q, k, v, scale = decode_inputs(B, H, L, D, seed)
    dq, dk, dv = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    dt = RF_F32 if out_dtype == torch.float32 else RF_BF16
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    o_ref = torch.empty(B, H, D, dtype=out_dtype, device="cuda")
    l_ref = torch.empty(B, H, device="cuda")
    need = int(lib.rf_attn_decode_workspace_size(B, H, L, D, nseg))
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    st = lib.rf_attn_decode(_ptr(dq), _ptr(dk), _ptr(dv), B, H, L, D, nseg, scale, dt, _ptr(o_ref), _ptr(l_ref),
                            _ptr(ws), need, stream)
    assert st == 0, lib.rf_last_error()
    # the no-allocation call gets fresh outputs filled with a sentinel
    o = torch.full((B, H, D), 7.0, dtype=out_dtype, device="cuda")
    lse = torch.full((B, H), 7.0, device="cuda")
    st = lib.rf_attn_decode_noalloc(_ptr(dq), _ptr(dk), _ptr(dv), B, H, L, D, nseg, scale, dt, _ptr(o), _ptr(lse),
                                    stream)
    assert st == 0, lib.rf_last_error()
    torch.cuda.synchronize()
    return o, lse, o_ref, l_ref


def test_noalloc_matches_workspace_call(rf):
    lib = rf.load()
    print("[noalloc] call 1: B=4 H=8 L=3000 D=128 nseg=16", flush=True)
    o1, l1, r1, rl1 = _run_both(lib, 4, 8, 3000, 128, 16, torch.bfloat16, 91)
    assert torch.equal(o1, r1) and torch.equal(l1, rl1)
    print("[noalloc] call 2: B=2 H=3 L=301 D=64 nseg=5", flush=True)
    o2, l2, r2, rl2 = _run_both(lib, 2, 3, 301, 64, 5, torch.float32, 92)
    assert torch.equal(o2, r2) and torch.equal(l2, rl2)
    assert np.isfinite(o2.cpu().numpy()).all()


def test_noalloc_single_segment_and_auto(rf):
    lib = rf.load()
    print("[noalloc] one segment and the library's segment choice", flush=True)
    o, l, r, rl = _run_both(lib, 2, 4, 700, 128, 1, torch.bfloat16, 93)
    assert torch.equal(o, r) and torch.equal(l, rl)
    o, l, r, rl = _run_both(lib, 1, 2, 5000, 64, 0, torch.bfloat16, 94)   # few rows: the rule splits
    assert torch.equal(o, r) and torch.equal(l, rl)


def test_noalloc_refuses_partials_beyond_the_scratch(rf):
    lib = rf.load()
    # 1024 rows x 1024 segments x 128 values x 4 bytes = 512 MiB of partials > the 32 MiB scratch;
    # refused on the host before any launch (the pointers are never dereferenced)
    p = 1 << 20
    st = lib.rf_attn_decode_noalloc(p, 2 * p, 3 * p, 32, 32, 4096, 128, 1024, 0.08, RF_BF16, 1 << 40,
                                    None, None)
    assert st == 2 and b"scratch" in lib.rf_last_error()
