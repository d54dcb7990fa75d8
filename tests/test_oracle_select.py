"""Pins of the oracle's router GEMV, top-k selection and routing weights.

Top-k is checked against a brute-force stable sort (numpy lexsort on
(index, -value)), exhaustively on tiny tie patterns and on 4000 random
tie-heavy logit sets (the PR #273 page checks its fused select against the
rank select over that many tie-heavy cases).  The softmax over the selected
logits is checked against closed forms; the router against numpy's matmul.
"""
import itertools

import numpy as np
import pytest


def brute_topk(logits, k):
    v = np.where(np.isnan(logits), -np.inf, logits.astype(np.float64))
    order = np.lexsort((np.arange(v.size), -v))   # value descending, then index ascending
    return order[:k].astype(np.int32)


def test_topk_exhaustive_tiny(orc):
    for E in range(1, 7):
        for vals in itertools.product([0.0, 1.0, 2.0], repeat=E):
            lg = np.array(vals, np.float32)
            for k in range(1, E + 1):
                assert np.array_equal(orc.topk(lg, k), brute_topk(lg, k)), (vals, k)


def test_topk_tie_heavy_4000(orc):
    rng = np.random.default_rng(273)
    for case in range(4000):
        E = int(rng.choice([8, 32, 64, 128, 256]))
        k = int(rng.integers(1, min(E, 16) + 1))
        levels = rng.standard_normal(int(rng.integers(1, 6))).astype(np.float32)
        lg = levels[rng.integers(0, levels.size, E)]
        if case % 5 == 0:           # sprinkle some distinct values among the ties
            lg = lg.copy()
            lg[rng.integers(0, E, 3)] = rng.standard_normal(3).astype(np.float32)
        assert np.array_equal(orc.topk(lg, k), brute_topk(lg, k)), case


def test_topk_special_values(orc):
    lg = np.zeros(256, np.float32)
    assert np.array_equal(orc.topk(lg, 8), np.arange(8))                    # all equal -> 0..k-1
    lg = np.arange(16, dtype=np.float32)[::-1].copy()
    assert np.array_equal(orc.topk(lg, 16), np.arange(16))                  # k = E: the stable sort
    lg = np.array([-0.0, 0.0, -1.0, 0.0], np.float32)                      # -0 and +0 tie
    assert np.array_equal(orc.topk(lg, 3), [0, 1, 3])
    lg = np.array([np.nan, -np.inf, 1.0, np.nan, -5.0], np.float32)        # NaN ranks as -inf
    assert np.array_equal(orc.topk(lg, 5), [2, 4, 0, 1, 3])
    # duplicated pairs (the tiny workload): the top pairs come out together, lower index first
    rng = np.random.default_rng(9)
    base = rng.standard_normal(16).astype(np.float32)
    lg = np.repeat(base, 2)
    ids = orc.topk(lg, 4)
    top2 = np.argsort(-base, kind="stable")[:2]
    assert np.array_equal(ids, [2 * top2[0], 2 * top2[0] + 1, 2 * top2[1], 2 * top2[1] + 1])


def test_softmax_closed_forms(orc):
    lg = np.array([0.3, -1.2, 2.5, 0.0], np.float32)
    # k = 1 -> weight 1
    assert orc.softmax_selected(lg, np.array([2], np.int32))[0] == 1.0
    # k = 2 -> w0 = sigmoid(l0 - l1)
    w = orc.softmax_selected(lg, np.array([2, 0], np.int32))
    d = float(lg[2]) - float(lg[0])
    assert w[0] == np.float32(1.0 / (1.0 + np.exp(-d)))
    assert np.isclose(w[1], np.float32(1.0 / (1.0 + np.exp(d))), rtol=2 ** -23, atol=0)
    # tied logits -> equal weights 1/k
    for k in (3, 4, 8):
        w = orc.softmax_selected(np.full(16, 0.7, np.float32), np.arange(k, dtype=np.int32))
        assert np.all(w == np.float32(1.0 / k))
    # random: weights sum to 1 and follow the logit order
    rng = np.random.default_rng(10)
    for _ in range(200):
        lg = rng.standard_normal(256).astype(np.float32) * 3
        ids = orc.topk(lg, 8)
        w = orc.softmax_selected(lg, ids)
        assert abs(float(w.astype(np.float64).sum()) - 1.0) < 1e-6
        assert np.all(np.diff(w) <= 0)
        # invariance to a common shift of the logits (up to fp32 rounding of w)
        w2 = orc.softmax_selected(lg + np.float32(4.0), ids)
        assert np.allclose(w, w2, rtol=1e-5, atol=0)


def test_router_matches_numpy_matmul(orc):
    rng = np.random.default_rng(11)
    W = (rng.standard_normal((256, 2048)) * 0.02).astype(np.float32)
    W[1] = W[0]                                     # duplicated row -> identical logit
    xn = rng.standard_normal(2048).astype(np.float32)
    got = orc.router(xn, W)
    want = (W.astype(np.float64) @ xn.astype(np.float64)).astype(np.float32)
    # fp64 accumulation of exact fp32 products: both round to the same fp32 except
    # within a few fp64 ulps of an fp32 rounding boundary
    assert np.sum(got != want) <= 2
    assert np.allclose(got, want, rtol=2 ** -23, atol=0)
    assert got[0] == got[1]
