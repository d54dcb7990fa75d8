"""Helpers of the GPU parity tests: device-side inputs, host copies for the
oracle, and the output criterion.

Criterion for a bf16 output (the 2e-3 bar, fp32 accumulate / bf16 output):
the GPU value must be the bf16 rounding of some real number within
2e-3 * max(|r|, 1e-3 * max|r|) of the oracle's unrounded value r.  bf16
rounding alone moves a value by up to 2^-9 (1.95e-3) relative, so comparing a
bf16 output to r with a plain relative bound could only ever pass by luck;
this form allows exactly one rounding on top of an fp32-accurate result.  The
floor (1e-3 of the largest magnitude) covers elements that cancel to almost
zero, where a relative bound is meaningless.  fp32 intermediates use the same
relative bound directly.
"""
import numpy as np
import torch

REL = 2e-3
FLOOR = 1e-3


def bf16_bits_to_f64(u16):
    return (np.asarray(u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_value(x):
    t = torch.from_numpy(np.asarray(x, np.float64).astype(np.float32)).to(torch.bfloat16)
    return t.to(torch.float64).numpy()


def bf16_within(gpu_u16, exact, rel=REL, floor=FLOOR):
    """(ok mask, allowed tolerance) for bf16 outputs against fp64 exact values."""
    r = np.asarray(exact, np.float64)
    scale = np.max(np.abs(r)) if r.size else 0.0
    tol = rel * np.maximum(np.abs(r), floor * scale)
    lo = f64_to_bf16_value(r - tol)
    hi = f64_to_bf16_value(r + tol)
    g = bf16_bits_to_f64(gpu_u16)
    return (g >= lo) & (g <= hi), tol


def assert_bf16_within(gpu_u16, exact, what="", rel=REL, floor=FLOOR):
    ok, tol = bf16_within(gpu_u16, exact, rel, floor)
    if not ok.all():
        i = np.flatnonzero(~ok)[:5]
        g = bf16_bits_to_f64(gpu_u16).ravel()
        r = np.asarray(exact, np.float64).ravel()
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} bf16 outputs outside the bound; "
                             f"flat idx {i.tolist()} gpu {g[i].tolist()} exact {r[i].tolist()} "
                             f"allowed {np.asarray(tol).ravel()[i].tolist()}")


def assert_f32_within(gpu, ref, what="", rel=REL, floor=FLOOR):
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    scale = np.max(np.abs(r)) if r.size else 0.0
    tol = rel * np.maximum(np.abs(r), floor * scale)
    bad = np.abs(g - r) > tol
    if bad.any():
        i = np.flatnonzero(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} fp32 values outside the bound; "
                             f"flat idx {i.tolist()} gpu {g.ravel()[i].tolist()} ref {r.ravel()[i].tolist()}")


def ulp_diff_f32(a, b):
    """|ulp distance| between two float32 arrays (same sign assumed for nonzero)."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def host(t):
    return t.detach().cpu().contiguous().numpy()


def u16_host(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.uint16).view(np.int16)).cuda().view(torch.bfloat16)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)
