"""Pins of the oracle's grouped batch path (several tokens, experts grouped).

Reading of the batch > 1 step: the tokens whose top-k holds expert e form its
group and the shared expert is one group of all tokens; each member gets
exactly what the batch-1 path gives it.  Pinned by: every token's outputs
equal a batch-1 layer call on that token alone (bit for bit), the reported
group sizes equal a count of the ids done here, the result does not depend on
which other tokens share the batch (a token's outputs are the same in a batch
of 3 and of 6), and the routed output is the slot-ordered weighted sum of the
per-slot expert outputs.  The batch inputs' steering is checked to put the two
chosen experts at the top of every steered token.
"""
import numpy as np
import torch

import workloads as wl

SMALL = wl.Config("small", H=512, E=16, k=4, F=128, Fs=128, router_dup=2, config_index=9)


def _batch_inputs(cfg, n):
    res = torch.stack([wl.randn((cfg.H,), wl.seed_for(9, 0, wl.T_INPUT, t)) for t in range(n)]).to(torch.bfloat16)
    rp = torch.stack([wl.randn((cfg.H,), wl.seed_for(9, 0, wl.T_RPREV, t)) for t in range(n)]).to(torch.bfloat16)
    sp = torch.stack([wl.randn((cfg.H,), wl.seed_for(9, 0, wl.T_SPREV, t)) for t in range(n)]).to(torch.bfloat16)
    return wl.u16(res), wl.u16(rp), wl.u16(sp)


def test_batch_is_the_single_token_path(orc):
    cfg = SMALL
    W = wl.to_numpy_weights(wl.layer_weights(cfg, 0, "cpu"))
    d = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs, eps=cfg.eps)
    n = 6
    res, rp, sp = _batch_inputs(cfg, n)
    ob = orc.moe_layer_batch(d, W, n, residual=res, routed_prev=rp, shared_prev=sp)
    for t in range(n):
        o1 = orc.moe_layer(d, W, residual=res[t], routed_prev=rp[t], shared_prev=sp[t])
        for key in ("out_sum", "xn", "xq", "ids", "weights", "h", "hs", "y", "ys", "routed", "shared",
                    "routed_exact", "shared_exact"):
            assert np.array_equal(np.asarray(o1[key]).reshape(-1), np.asarray(ob[key][t]).reshape(-1)), (t, key)
        assert ob["shared_gate"][t] == o1["shared_gate"][0]
    # duplicated router rows: experts come in tied pairs, so groups of two or more exist
    ids = ob["ids"]
    for t in range(n):
        for s in range(cfg.k):
            assert ob["group_size"][t][s] == int(np.sum(ids == ids[t][s]))
    assert ob["group_size"].max() >= 2
    # combine: slot-ordered weighted sum of the per-slot outputs
    for t in range(n):
        acc = np.zeros(cfg.H)
        for s in range(cfg.k):
            acc += ob["weights"][t][s].astype(np.float64) * ob["y"][t][s].astype(np.float64)
        assert np.array_equal(ob["routed_exact"][t], acc)


def test_batch_result_does_not_depend_on_the_batch(orc):
    cfg = SMALL
    W = wl.to_numpy_weights(wl.layer_weights(cfg, 0, "cpu"))
    d = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs, eps=cfg.eps)
    res, rp, sp = _batch_inputs(cfg, 6)
    big = orc.moe_layer_batch(d, W, 6, residual=res, routed_prev=rp, shared_prev=sp)
    sub = [1, 4, 5]
    small = orc.moe_layer_batch(d, W, 3, residual=res[sub], routed_prev=rp[sub], shared_prev=sp[sub])
    for j, t in enumerate(sub):
        for key in ("ids", "h", "y", "routed", "shared"):
            assert np.array_equal(big[key][t], small[key][j]), (t, key)


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
