"""Pins of the oracle's grouped batch path (several tokens, experts grouped).

The bf16 path of a row is pinned against the independent numpy decoders with
a bf16 rounding written here from the format's definition: the same value up
to the order of an fp64 sum (compared to one fp32 ulp).  An exact closed form
(weights and activations that are small integers, so nothing rounds) and the
bf16 error bound against the dense fp64 product pin its definition.  The
grouping is pinned by the threshold switch: groups below the threshold equal
the single-token integer path exactly, groups at or above it follow the bf16
pipeline rebuilt here in numpy.  The batch inputs' steering is checked to
put the two chosen experts at the top of every steered token.
"""
import numpy as np
import pytest
import torch

import qformats as qf
import workloads as wl


def bf16_round(x):
    """fp32 -> bf16 (round to nearest, ties to even) -> fp64, vectorised numpy."""
    u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> 16
    drop = u & 0xFFFF
    up = (drop > 0x8000) | ((drop == 0x8000) & ((keep & 1) == 1))
    keep = (keep + up.astype(np.uint64)) & 0xFFFF
    return (keep.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _row(typ, K, seed, std=0.02):
    x = wl.randn((1, K), seed, "cpu", std)
    return wl.quantize(x, typ).numpy().reshape(-1)


def _x(K, seed):
    return wl.randn((K,), seed, "cpu").numpy().astype(np.float32)


@pytest.mark.parametrize("typ", [wl.Q4_K, wl.Q5_K, wl.Q8_0])
@pytest.mark.parametrize("n_active", [None, 100])
def test_row_dot_bf16_matches_numpy(orc, typ, n_active):
    K = 512
    for seed in range(6):
        row = _row(typ, K, 1000 + seed)
        x = _x(K, 2000 + seed)
        n = K if n_active is None else n_active
        w = qf.decode(row, typ)
        wb = bf16_round(w.astype(np.float32))          # f32(w) then bf16
        xb = bf16_round(x)
        ref = np.float32(np.dot(wb[:n], xb[:n]))
        got = np.float32(orc.row_dot_bf16(row, typ, K, x, n))
        assert abs(float(got) - float(ref)) <= float(np.spacing(abs(ref))), (seed, got, ref)


def test_rows_dot_bf16_is_the_single_row_dot(orc):
    K, n_rows = 512, 7
    rows = wl.quantize(wl.randn((n_rows, K), 77) * 0.02, wl.Q5_K).numpy()
    x = np.random.default_rng(3).standard_normal((4, 300)).astype(np.float32)
    rb = wl.row_bytes(wl.Q5_K, K)
    got = orc.rows_dot_bf16(rows, wl.Q5_K, K, n_rows, x)
    for j in range(4):
        for r in range(n_rows):
            assert got[j, r] == np.float32(orc.row_dot_bf16(rows.reshape(n_rows, rb)[r], wl.Q5_K, K, x[j], 300))


def test_row_dot_bf16_exact_on_small_integers(orc):
    """d = 1, dmin = 0, scales 1..3, codes 0..15: every weight and activation is a
    small integer, so no rounding happens anywhere and the result is the integer dot."""
    K = 256
    rng = np.random.default_rng(7)
    sc = rng.integers(1, 4, 8)
    m = np.zeros(8, np.int64)
    q = rng.integers(0, 16, 256)
    blk = wl.assemble_kquant(torch.tensor([1.0]), torch.tensor([0.0]), torch.tensor(sc[None]),
                             torch.tensor(m[None]), torch.tensor(q[None]), wl.Q4_K).numpy().reshape(-1)
    w = qf.decode(blk, wl.Q4_K)
    assert np.array_equal(w, np.repeat(sc, 32) * q)
    x = rng.integers(-20, 21, K).astype(np.float32)
    assert orc.row_dot_bf16(blk, wl.Q4_K, K, x) == float(np.dot(w, x))


@pytest.mark.parametrize("typ", [wl.Q4_K, wl.Q8_0])
def test_row_dot_bf16_error_bound(orc, typ):
    """|bf16 path - exact dense product| <= sum|w x| * (2^-8 + 2^-17) + |exact| * 2^-23:
    each operand rounds to bf16 with relative error <= 2^-9."""
    K = 1024
    for seed in range(8):
        row = _row(typ, K, 3000 + seed)
        x = _x(K, 4000 + seed)
        w = qf.decode(row, typ)
        exact = float(np.dot(w, x.astype(np.float64)))
        bound = float(np.abs(w) @ np.abs(x.astype(np.float64))) * (2.0 ** -8 + 2.0 ** -17) + abs(exact) * 2.0 ** -23
        assert abs(orc.row_dot_bf16(row, typ, K, x) - exact) <= bound


SMALL = wl.Config("small", H=512, E=16, k=4, F=128, Fs=128, router_dup=2, config_index=9)


def _batch_inputs(cfg, n):
    res = torch.stack([wl.randn((cfg.H,), wl.seed_for(9, 0, wl.T_INPUT, t)) for t in range(n)]).to(torch.bfloat16)
    rp = torch.stack([wl.randn((cfg.H,), wl.seed_for(9, 0, wl.T_RPREV, t)) for t in range(n)]).to(torch.bfloat16)
    sp = torch.stack([wl.randn((cfg.H,), wl.seed_for(9, 0, wl.T_SPREV, t)) for t in range(n)]).to(torch.bfloat16)
    return wl.u16(res), wl.u16(rp), wl.u16(sp)


def _silu(x):
    return x / (1.0 + np.exp(-x))


def test_batch_below_threshold_is_the_single_token_path(orc):
    cfg = SMALL
    W = wl.to_numpy_weights(wl.layer_weights(cfg, 0, "cpu"))
    d = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs, eps=cfg.eps)
    n = 5
    res, rp, sp = _batch_inputs(cfg, n)
    ob = orc.moe_layer_batch(d, W, n, threshold=n + 1, residual=res, routed_prev=rp, shared_prev=sp)
    for t in range(n):
        o1 = orc.moe_layer(d, W, residual=res[t], routed_prev=rp[t], shared_prev=sp[t])
        for key in ("out_sum", "ids", "routed", "shared"):
            assert np.array_equal(o1[key], ob[key][t]), (t, key)
        assert np.array_equal(o1["y"], ob["y"][t])


def test_batch_grouped_path_rebuilt_in_numpy(orc):
    """threshold 2 with duplicated router rows: paired experts form groups of >= 2.
    Those slots must follow the bf16 pipeline (rebuilt here from the numpy
    decoders and bf16_round), the others the single-token integer path."""
    cfg = SMALL
    W = wl.to_numpy_weights(wl.layer_weights(cfg, 0, "cpu"))
    d = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs, eps=cfg.eps)
    n = 6
    res, rp, sp = _batch_inputs(cfg, n)
    thr = 2
    ob = orc.moe_layer_batch(d, W, n, threshold=thr, residual=res, routed_prev=rp, shared_prev=sp)
    H, F = cfg.H, cfg.F
    rb_gu, rb_dn = wl.row_bytes(wl.Q4_K, H), wl.row_bytes(wl.Q4_K, wl.pad_k(wl.Q4_K, F))
    Kp = wl.pad_k(wl.Q4_K, F)
    grouped = 0
    for t in range(n):
        o1 = orc.moe_layer(d, W, residual=res[t], routed_prev=rp[t], shared_prev=sp[t])
        xb = bf16_round(ob["xn"][t])
        for s in range(cfg.k):
            e = int(ob["ids"][t][s])
            count = int(np.sum(ob["ids"] == e))
            assert ob["group_size"][t][s] == count
            if count < thr:
                assert np.array_equal(ob["y"][t][s], o1["y"][s]), (t, s)
                continue
            grouped += 1
            G = bf16_round(qf.matrix(W["gate"].reshape(cfg.E, -1)[e], wl.Q4_K, F, H).astype(np.float32))
            U = bf16_round(qf.matrix(W["up"].reshape(cfg.E, -1)[e], wl.Q4_K, F, H).astype(np.float32))
            D = bf16_round(qf.matrix(W["down"].reshape(cfg.E, -1)[e], wl.Q4_K, H, Kp).astype(np.float32))
            g = (G @ xb).astype(np.float32)
            u = (U @ xb).astype(np.float32)
            h = (_silu(g.astype(np.float64)) * u.astype(np.float64)).astype(np.float32)
            np.testing.assert_allclose(ob["h"][t][s], h, rtol=1e-5, atol=1e-9)
            hb = np.zeros(Kp)
            hb[:F] = bf16_round(ob["h"][t][s])
            y = (D @ hb).astype(np.float32)
            np.testing.assert_allclose(ob["y"][t][s], y, rtol=1e-5, atol=1e-7)
    assert grouped > 0
    # the shared expert is one group of all n >= thr tokens: bf16 path too
    G = bf16_round(qf.matrix(W["sgate"], wl.Q4_K, cfg.Fs, H).astype(np.float32))
    U = bf16_round(qf.matrix(W["sup"], wl.Q4_K, cfg.Fs, H).astype(np.float32))
    for t in range(n):
        xb = bf16_round(ob["xn"][t])
        g = (G @ xb).astype(np.float32)
        u = (U @ xb).astype(np.float32)
        h = (_silu(g.astype(np.float64)) * u.astype(np.float64)).astype(np.float32)
        np.testing.assert_allclose(ob["hs"][t], h, rtol=1e-5, atol=1e-9)
    # combine in slot order, one rounding
    for t in range(n):
        acc = np.zeros(H)
        for s in range(cfg.k):
            acc += ob["weights"][t][s].astype(np.float64) * ob["y"][t][s].astype(np.float64)
        np.testing.assert_allclose(ob["routed_exact"][t], acc, rtol=1e-12, atol=1e-15)


def test_batch_inputs_steer_the_chosen_pair(orc):
    cfg = wl.CONFIGS["batch"]
    w = wl.rand_uniform((cfg.H,), wl.seed_for(cfg.config_index, 0, wl.T_NORM), 0.5, 1.5).numpy()
    R = wl._router_rows(cfg, 0, "cpu").numpy()
    for n in (8, 32):
        inp, steer, (a, b) = wl.batch_inputs(cfg, n)
        assert len(steer) == n // 4 and a < b
        for t in steer:
            o = orc.add_rmsnorm(wl.u16(inp["residual"][t]), wl.u16(inp["routed_prev"][t]),
                                wl.u16(inp["shared_prev"][t]), w, cfg.eps)
            xn = o[1] if isinstance(o, tuple) else o["xn"]
            assert set(orc.topk(orc.router(xn, R), 2).tolist()) == {a, b}, (n, t)
