"""Helpers for the GPU parity tests: moving seeded inputs to the device and
comparing results with the oracle under a stated tolerance."""
import numpy as np
import torch


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).cuda()


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def host(t):
    """Device tensor -> float64 numpy (bf16 decoded exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy().astype(np.float64) if t.dtype.is_floating_point else t.cpu().numpy()


def assert_close(got, ref, atol, rtol, what):
    """Pass iff |got - ref| <= atol + rtol * |ref| elementwise; reports max errors and failures."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    same_inf = np.isinf(ref) & (got == ref)
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(got - ref))
    bad = ~(err <= atol + rtol * np.abs(ref))
    if bad.any():
        i = np.unravel_index(np.argmax(np.where(bad, err, -1)), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
                             f"(atol={atol}, rtol={rtol}); max abs err {np.nanmax(err):.3g}; "
                             f"worst at {i}: got {got[i]!r} ref {ref[i]!r}")
    return float(np.max(err)) if err.size else 0.0
