"""Pins of the oracle's residual-add + RMSNorm (+ Q8_1) step.

Against closed forms (zero, constant and two-level vectors), power-of-two
scale invariance, the fold identity of the PR #273 page (the 3-input fold is
bit-identical to the separate residual add followed by the 2-input norm),
and the reductions of the 2-input / no-previous-output forms.
"""
import numpy as np
import torch


def bf16(x):
    return torch.tensor(np.asarray(x, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f64(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


H = 2048


def test_zero_vector(orc):
    out_sum, xn, xq = orc.add_rmsnorm(np.zeros(H, np.uint16), None, None, np.ones(H, np.float32), 1e-6)
    assert not out_sum.any() and not xn.any() and not xq.any()


def test_constant_vector_closed_form(orc):
    w = np.random.default_rng(1).uniform(0.5, 1.5, H).astype(np.float32)
    for c in (1.0, -3.0, 0.0078125, 200.0):
        res = bf16(np.full(H, c))
        _, xn, _ = orc.add_rmsnorm(res, None, None, w, 1e-6)
        cv = f64(res)[0]
        want = (cv / np.sqrt(cv * cv + np.float64(np.float32(1e-6)))) * w.astype(np.float64)
        assert np.array_equal(xn, want.astype(np.float32)) or np.allclose(xn, want, rtol=2 ** -23, atol=0)
        if abs(c) >= 1.0:
            assert np.allclose(xn, np.sign(c) * w, rtol=1e-5)


def test_two_level_vector_closed_form(orc):
    # u = [3, 4, 3, 4, ...] -> mean(u^2) = 12.5 exactly
    u = np.tile([3.0, 4.0], H // 2)
    _, xn, _ = orc.add_rmsnorm(bf16(u), None, None, np.ones(H, np.float32), 1e-6)
    r = 1.0 / np.sqrt(12.5 + np.float64(np.float32(1e-6)))
    assert xn[0] == np.float32(3.0 * r) and xn[1] == np.float32(4.0 * r)


def test_power_of_two_scale_invariance(orc):
    rng = np.random.default_rng(2)
    res = bf16(rng.standard_normal(H))
    w = rng.uniform(0.5, 1.5, H).astype(np.float32)
    _, xn1, xq1 = orc.add_rmsnorm(res, None, None, w, 0.0)
    res4 = bf16(f64(res) * 4.0)
    _, xn4, xq4 = orc.add_rmsnorm(res4, None, None, w, 0.0)
    assert np.array_equal(xn1, xn4) and np.array_equal(xq1, xq4)


def test_fold_identity(orc):
    """add_rmsnorm3(res, routed, shared) == add_rmsnorm2(res, bf16(routed + shared)), bitwise."""
    rng = np.random.default_rng(3)
    w = rng.uniform(0.5, 1.5, H).astype(np.float32)
    for t in range(20):
        res, rt, sh = (bf16(rng.standard_normal(H) * s) for s in (1.0, 0.3, 0.1))
        a = orc.add_rmsnorm(res, rt, sh, w, 1e-6)
        t_ = bf16(f64(rt) + f64(sh))          # the separate residual_add (bf16 output)
        b = orc.add_rmsnorm(res, t_, None, w, 1e-6)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)
        # out_sum is the bf16 of residual + t
        assert np.array_equal(a[0], bf16(f64(res) + f64(t_)))


def test_two_input_and_empty_forms(orc):
    rng = np.random.default_rng(4)
    w = rng.uniform(0.5, 1.5, H).astype(np.float32)
    res = bf16(rng.standard_normal(H))
    z = np.zeros(H, np.uint16)
    a = orc.add_rmsnorm(res, None, None, w, 1e-6)
    b = orc.add_rmsnorm(res, z, None, w, 1e-6)
    c = orc.add_rmsnorm(res, z, z, w, 1e-6)
    for x, y, v in zip(a, b, c):
        assert np.array_equal(x, y) and np.array_equal(x, v)
    assert np.array_equal(a[0], res)       # no previous output: the residual passes through


def test_norm_output_is_unit_rms(orc):
    rng = np.random.default_rng(5)
    res = bf16(rng.standard_normal(H) * 7)
    _, xn, xq = orc.add_rmsnorm(res, None, None, np.ones(H, np.float32), 1e-6)
    assert abs(np.sqrt(np.mean(xn.astype(np.float64) ** 2)) - 1.0) < 1e-6
    # xq is the Q8_1 of xn
    assert np.array_equal(xq, orc.quantize_q8_1(xn))
