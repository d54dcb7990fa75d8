"""Pins of the oracle's load-time requantisation to Q4_K (Q8_0 / Q5_K / Q4_K
source rows -> Q4_K rows).

The quantiser is pinned to an independent implementation of the same
min/max rule (the torch one that generates the test weights, written
separately in vectorised form), to a closed form (blocks on a full grid come
back unchanged), and to its error bound on random data.  The source decode
and the row/superblock walk are pinned to the numpy decoders.
"""
import numpy as np
import pytest
import torch

import qformats as qf
import workloads as wl


def _blocks_x(n_sb, seed):
    """fp32 superblocks with sub-blocks of mixed character: signed, all
    positive, all negative, all zero, one value, wide scale range."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_sb, 8, 32)).astype(np.float64)
    kind = rng.integers(0, 8, (n_sb, 8))
    x[kind == 1] = np.abs(x[kind == 1])
    x[kind == 2] = -np.abs(x[kind == 2])
    x[kind == 3] = 0.0
    x[kind == 4, 1:] = 0.0
    x *= np.exp2(rng.integers(-12, 6, (n_sb, 1, 1)))
    return x.astype(np.float32).reshape(n_sb, 256)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_quantize_q4k_matches_the_torch_rule(orc, seed):
    x = _blocks_x(64, seed)
    ref = wl.quantize_kquant(torch.from_numpy(x), wl.Q4_K).numpy().reshape(-1)
    got = orc.quantize_q4k(x)
    assert np.array_equal(got, ref)


def test_quantize_q4k_full_grid_blocks_come_back_unchanged(orc):
    """Sub-block j holds d*sc_j*q - dmin*m_j for every q in 0..15 (twice), with
    sc and m reaching 63 somewhere: the rule recovers d, dmin, sc, m and q."""
    rng = np.random.default_rng(11)
    for trial in range(20):
        d = float(np.exp2(rng.integers(-14, -4)))
        dmin = float(np.exp2(rng.integers(-14, -4)))
        sc = rng.integers(1, 64, 8)
        m = rng.integers(0, 64, 8)
        sc[rng.integers(0, 8)] = 63
        m[rng.integers(0, 8)] = 63
        q = np.tile(np.arange(16), (8, 2))
        for j in range(8):
            rng.shuffle(q[j])
        x = (d * sc[:, None] * q - dmin * m[:, None]).astype(np.float32).reshape(256)
        blk = orc.quantize_q4k(x).reshape(1, 144)
        d2, dmin2, sc2, m2 = qf.kquant_fields(blk)
        assert d2[0] == d and dmin2[0] == dmin, trial
        assert np.array_equal(sc2[0], sc) and np.array_equal(m2[0], m), trial
        assert np.array_equal(qf.kquant_codes(blk, qf.Q4_K)[0], q.reshape(256)), trial


@pytest.mark.parametrize("seed", [4, 5])
def test_quantize_q4k_error_bound(orc, seed):
    """Each value comes back within half its sub-block step, plus what the
    6-bit scale/min rounding moves the sub-block's range by."""
    x = _blocks_x(128, seed).astype(np.float64)
    blk = orc.quantize_q4k(x.astype(np.float32)).reshape(-1, 144)
    xr = qf.decode(blk.reshape(-1), qf.Q4_K).reshape(x.shape)
    d, dmin, sc, m = qf.kquant_fields(blk)
    xs = x.reshape(-1, 8, 32)
    lo = np.minimum(xs.min(-1), 0.0)
    step = (xs.max(-1) - lo) / 15.0
    es = d[:, None] * sc
    eo = dmin[:, None] * m
    bound = 0.5 * es + 15.0 * np.abs(step - es) + np.abs(-lo - eo) + 1e-6 * np.abs(xs).max(-1)
    err = np.abs(xr.reshape(-1, 8, 32) - xs).max(-1)
    assert (err <= bound + 1e-12).all(), float((err - bound).max())
    # and the error is small against the sub-block range in the normal case
    ok = step > 0
    assert np.median(err[ok] / (step[ok] * 15.0)) < 0.05


@pytest.mark.parametrize("src_type", [wl.Q8_0, wl.Q5_K, wl.Q4_K])
def test_requant_rows_decode_then_quantise(orc, src_type):
    n_rows, K = 5, 768
    x = torch.from_numpy(_blocks_x(n_rows * K // 256, 7 + src_type).reshape(n_rows, K))
    src = wl.quantize(x, src_type).numpy()
    got = orc.requant_q4k(src, src_type, n_rows, K)
    dec = qf.decode(src.reshape(-1), src_type).reshape(n_rows, K).astype(np.float32)
    ref = orc.quantize_q4k(dec)
    assert np.array_equal(got, ref)
