"""Checks of an L-layer stack's per-layer outputs against the oracle, shared
by the persistent-kernel and per-layer-kernel stack tests.

Per token the stack under test writes every layer's selection, residual
(out_sum), routed and shared outputs.  Each layer is checked two ways:

  stage-isolated: the oracle runs the layer on the GPU's own inputs to it
    (the GPU's previous residual, routed and shared outputs).  Its top-k must
    be the GPU's selection exactly; the fold (out_sum) must be bit-exact; the
    routed and shared bf16 outputs must meet the strict criterion (each the
    bf16 rounding of a value within 2e-3 relative of the oracle's unrounded
    value).  A selection difference here can only come from a last-bit
    difference of two logits (both sides sum in fp64 and round to fp32): it
    is allowed only within 4 fp32 ulps of the logits and counted.
  chained: the oracle runs its own chain from the token input.  Where its
    selection differs from the GPU's, the difference must be a near tie: the
    GPU's selection must be a valid top-k of the oracle's logits once every
    logit may move by delta_e = H * 2^-24 * sum_i |W_ei * xn_i| (the fp32
    rounding bound of a dot product of length H); the oracle then continues
    with the GPU's selection and the event is counted.  out_sum, routed and
    shared must stay within a relative L2 distance of 2e-3 of the oracle's at
    every layer, and so must the stack output; the largest max-norm error per
    layer is printed, so its growth over the layers is on record.  When the
    two chains stay bit-identical the stack output must also meet the strict
    criterion.
"""
import numpy as np
import torch

import gpu_util as gu
import workloads as wl


def _rel_l2(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    n = np.linalg.norm(r)
    return float(np.linalg.norm(g - r) / n) if n > 0 else float(np.linalg.norm(g))


def _max_rel(g, r):
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    m = np.max(np.abs(r))
    return float(np.max(np.abs(g - r)) / m) if m > 0 else float(np.max(np.abs(g)))


def _near_tie_ok(sel, logits, delta):
    """sel (k ids, slot order) is a top-k of `logits` once each logit may move by delta."""
    lg = np.asarray(logits, np.float64)
    sel = [int(e) for e in sel]
    rest = np.setdiff1d(np.arange(lg.size), sel)
    for s, a in enumerate(sel):
        if rest.size and np.any(lg[rest] - delta[rest] > lg[a] + delta[a]):
            return False
        for b in sel[s + 1:]:
            if lg[b] - delta[b] > lg[a] + delta[a]:
                return False
    return True


def _router_delta(W, xn, H, ulps):
    return ulps * 2.0 ** -24 * (np.abs(W.astype(np.float64)) @ np.abs(np.asarray(xn, np.float64)))


def _f64(u16):
    return gu.bf16_bits_to_f64(u16)


def _fold(res, rt, sh, has_shared):
    """bf16(res + bf16(rt + sh)) (or bf16(res + rt)) on bf16 bit patterns."""
    b = lambda v: gu.u16_host(torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16))
    t = b(_f64(rt) + _f64(sh)) if has_shared else np.asarray(rt, np.uint16)
    return b(_f64(res) + _f64(t))


def run_and_check(q, orc, cfg, st, dt, tokens, mode, with_attn=False):
    """with_attn: every layer runs behind a seeded attention-block output
    (u1 = the fold of the previous outputs, then the 2-input add-norm of
    (u1, attn_l)); the oracle's layer then takes (u1, attn_l) as its inputs."""
    L, H, E, k = cfg.layers, cfg.H, cfg.E, cfg.k
    has_sh = cfg.Fs > 0
    Ws = [wl.layer_weights(cfg, l, "cuda", shared_type=st, down_type=dt) for l in range(L)]
    Wn = [wl.to_numpy_weights(w) for w in Ws]
    desc_g = q.make_desc(H, E, k, cfg.F, cfg.Fs, down_type=dt, shared_type=st, eps=cfg.eps)
    desc_o = orc.make_desc(H, E, k, cfg.F, cfg.Fs, down_type=dt, shared_type=st, eps=cfg.eps)
    ws = q.alloc_workspace(desc_g, L)
    persistent = mode == q.MOE_STACK_PERSISTENT
    if persistent:
        q.moe_stack_bind(desc_g, Ws, ws)
    arr = q.layer_array(Ws)
    events = {"chained near ties": 0, "isolated last-bit ties": 0, "layers bit-identical": 0, "layers": 0}
    growth = np.zeros(L)
    for t in tokens:
        if t == "zero":
            inp = torch.zeros(H, dtype=torch.bfloat16)
        else:
            inp = wl.token_inputs(cfg, t, "cpu")["residual"]
        out = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
        ids = torch.full((L, k), -1, dtype=torch.int32, device="cuda")
        res = torch.zeros(L, H, dtype=torch.bfloat16, device="cuda")
        rts = torch.zeros(L, H, dtype=torch.bfloat16, device="cuda")
        shs = torch.zeros(L, H, dtype=torch.bfloat16, device="cuda") if has_sh else None
        at_t = None
        if with_attn:
            at_t = torch.stack([wl.attention_output(cfg, 0 if t == "zero" else t, l) for l in range(L)])
        q.moe_decode_stack(desc_g, None, inp.cuda(), out, ids, res, mode, ws, layer_array=arr,
                           routed_per_layer=rts, shared_per_layer=shs,
                           attn=None if at_t is None else at_t.cuda().contiguous())
        at_u = None if at_t is None else wl.u16(at_t)

        def oracle_layer(l, r_in, rt_in, sh_in, ids=None):
            if at_u is None:
                return orc.moe_layer(desc_o, Wn[l], r_in, rt_in, sh_in, ids=ids)
            u1 = r_in if rt_in is None else _fold(r_in, rt_in, sh_in, has_sh)
            return orc.moe_layer(desc_o, Wn[l], u1, at_u[l], None, ids=ids)
        torch.cuda.synchronize()
        if persistent:
            assert q.stack_status(desc_g, L, ws) == 0
        g_ids, g_res, g_rt = gu.host(ids), gu.u16_host(res), gu.u16_host(rts)
        g_sh = gu.u16_host(shs) if has_sh else None
        inp_u = wl.u16(inp)
        # ---- stage-isolated, layer by layer on the GPU's own inputs
        for l in range(L):
            r_in = inp_u if l == 0 else g_res[l - 1]
            rt_in = None if l == 0 else g_rt[l - 1]
            sh_in = None if (l == 0 or not has_sh) else g_sh[l - 1]
            o = oracle_layer(l, r_in, rt_in, sh_in)
            if not np.array_equal(o["ids"], g_ids[l]):
                d = _router_delta(Wn[l]["router_w"], o["xn"], H, 4.0)
                assert _near_tie_ok(g_ids[l], o["logits"], d), (t, l, o["ids"], g_ids[l])
                events["isolated last-bit ties"] += 1
                o = oracle_layer(l, r_in, rt_in, sh_in, ids=g_ids[l])
            assert np.array_equal(g_res[l], o["out_sum"]), (t, l, "out_sum")
            gu.assert_bf16_within(g_rt[l], o["routed_exact"], f"token {t} layer {l} routed")
            if has_sh:
                gu.assert_bf16_within(g_sh[l], o["shared_exact"], f"token {t} layer {l} shared")
        # ---- chained: the oracle's own chain
        r_o, rt_o, sh_o = inp_u, None, None
        identical = True
        for l in range(L):
            o = oracle_layer(l, r_o, rt_o, sh_o if has_sh else None)
            if not np.array_equal(o["ids"], g_ids[l]):
                d = _router_delta(Wn[l]["router_w"], o["xn"], H, float(H))
                assert _near_tie_ok(g_ids[l], o["logits"], d), (t, l, o["ids"], g_ids[l])
                events["chained near ties"] += 1
                o = oracle_layer(l, r_o, rt_o, sh_o if has_sh else None, ids=g_ids[l])
            pairs = [("out_sum", g_res[l], _f64(o["out_sum"])), ("routed", g_rt[l], o["routed_exact"])]
            if has_sh:
                pairs.append(("shared", g_sh[l], o["shared_exact"]))
            for name, g, r in pairs:
                e = _rel_l2(_f64(g), r)
                assert e <= gu.REL, (t, l, name, e)
                growth[l] = max(growth[l], _max_rel(_f64(g), r))
            same = np.array_equal(g_res[l], o["out_sum"]) and np.array_equal(g_rt[l], o["routed"]) and \
                (not has_sh or np.array_equal(g_sh[l], o["shared"]))
            events["layers bit-identical"] += int(same)
            events["layers"] += 1
            identical &= same
            r_o, rt_o, sh_o = o["out_sum"], o["routed"], o["shared"]
        o_out = _fold(r_o, rt_o, sh_o, has_sh)
        g_out = gu.u16_host(out)
        assert _rel_l2(_f64(g_out), _f64(o_out)) <= gu.REL
        # the fold of the GPU's own last layer is exact
        assert np.array_equal(g_out, _fold(g_res[L - 1], g_rt[L - 1], g_sh[L - 1] if has_sh else None, has_sh))
        if identical:
            exact = _f64(r_o) + (_f64(_fold(np.zeros(H, np.uint16), rt_o, sh_o, True)) if has_sh else _f64(rt_o))
            gu.assert_bf16_within(g_out, exact, f"token {t} stack output")
        if t == "zero":
            assert not g_out.any() and np.all(g_ids == np.arange(k))
        print(f"  token {t}: chains identical {identical}; output bits equal "
              f"{float((g_out == o_out).mean()):.5f}", flush=True)
    print(f"  {events}; max-norm error by layer (max over tokens): "
          + " ".join(f"{v:.1e}" for v in growth), flush=True)
    return Ws, desc_g, ws, arr
