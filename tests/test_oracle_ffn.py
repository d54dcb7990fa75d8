"""Pins of the oracle's expert FFN, layer and stack.

The FFN is checked stage by stage against a dense fp64 pipeline built from the
independent numpy decoders: g = G a, u = U a (a = decoded Q8_1 activations),
h = silu(g) * u, y = D deq(Q8_1(h)), routed = sum_s w_s y_s, shared =
sigmoid-gate * ys.  The only allowed differences are the fp16 rounding of the
stored Q8_1 sums (read by the K-quant min term) and the fp32 storage
roundings.  A swapped gate/up, a missing min term, a wrong sub-block pairing,
a dropped gate or a mis-ordered combine all exceed these bounds.
The layer and stack are checked to be exactly the composition of their
(separately pinned) steps.
"""
import numpy as np
import pytest
import torch

import qformats as qf
import workloads as wl


def _np_weights(cfg, layer=0, **kw):
    return wl.to_numpy_weights(wl.layer_weights(cfg, layer, "cpu", **kw))


def _minterm_bound(blob, typ, rows, K, xq):
    """Per-row bound sum_j dmin*m_j*|s_j - d_j*sum(q_j)| of the stored-sum rounding."""
    if typ == qf.Q8_0:
        return np.zeros(rows)
    nb = qf.NB[typ]
    _, dmin, _, m = qf.kquant_fields(np.asarray(blob, np.uint8).reshape(-1, nb))
    mins = (dmin[:, None] * m).reshape(rows, K // 32)
    da, sa, qa = qf.q8_fields(xq, qf.Q8_1)
    return mins @ np.abs(sa - da * qa.sum(1))


def _silu(x):
    return x / (1.0 + np.exp(-x))


def _check_expert(orc, gate_blob, up_blob, down_blob, gu_type, dn_type, H, F, xq, h_or, y_or):
    Kp = wl.pad_k(dn_type, F)
    G = qf.matrix(gate_blob, gu_type, F, H)
    U = qf.matrix(up_blob, gu_type, F, H)
    da, _, qa = qf.q8_fields(xq, qf.Q8_1)
    a = (da[:, None] * qa).reshape(-1)
    g, u = G @ a, U @ a
    bg = _minterm_bound(gate_blob, gu_type, F, H, xq) + 1e-12 * (np.abs(G) @ np.abs(a))
    bu = _minterm_bound(up_blob, gu_type, F, H, xq) + 1e-12 * (np.abs(U) @ np.abs(a))
    # f32 storage of g and u, then of h
    bg += np.abs(g) * 2.0 ** -24
    bu += np.abs(u) * 2.0 ** -24
    h = _silu(g) * u
    bh = 1.1 * bg * (np.abs(u) + bu) + np.abs(_silu(g)) * bu + np.abs(h) * 2.0 ** -23
    assert np.all(np.abs(h_or - h) <= bh), np.max(np.abs(h_or - h) - bh)
    # down: against the decoded Q8_1 of the oracle's own h (zero blocks pad F up to Kp)
    hpad = np.zeros(Kp, np.float32)
    hpad[:F] = h_or
    hq = orc.quantize_q8_1(hpad[:F])
    hq = np.concatenate([hq, np.zeros((Kp - F) // 32 * 36, np.uint8)])
    D = qf.matrix(down_blob, dn_type, H, Kp)
    dh, _, qh = qf.q8_fields(hq, qf.Q8_1)
    ah = (dh[:, None] * qh).reshape(-1)
    y = D @ ah
    by = _minterm_bound(down_blob, dn_type, H, Kp, hq) + 1e-12 * (np.abs(D) @ np.abs(ah)) + np.abs(y) * 2.0 ** -24
    assert np.all(np.abs(y_or - y) <= by), np.max(np.abs(y_or - y) - by)
    # gate and up are not interchangeable on this data (the check above would catch a swap)
    assert np.max(np.abs(_silu(u) * g - h)) > 100 * np.max(bh)


@pytest.mark.parametrize("shared_type,down_type", [(wl.Q4_K, wl.Q4_K), (wl.Q8_0, wl.Q5_K)])
def test_expert_ffn_dense_reference(orc, shared_type, down_type):
    cfg = wl.CONFIGS["tiny"]
    W = _np_weights(cfg, shared_type=shared_type, down_type=down_type)
    H, F, Fs, k = cfg.H, cfg.F, cfg.Fs, cfg.k
    x = np.random.default_rng(12).standard_normal(H).astype(np.float32)
    xq = orc.quantize_q8_1(x)
    ids = np.array([3, 17, 5, 30], np.int32)
    wts = np.array([0.4, 0.3, 0.2, 0.1], np.float32)
    sg = np.float32(0.37)
    desc = orc.make_desc(H, cfg.E, k, F, Fs, down_type=down_type, shared_type=shared_type, norm=0)
    o = orc.expert_ffn(desc, W, xq, ids, wts, float(sg))
    gu_rb, dn_rb = wl.row_bytes(wl.Q4_K, H), wl.row_bytes(down_type, wl.pad_k(down_type, F))
    for s, e in enumerate(ids):
        _check_expert(orc, W["gate"][e].ravel(), W["up"][e].ravel(), W["down"][e].ravel(),
                      wl.Q4_K, down_type, H, F, xq, o["h"][s].astype(np.float64), o["y"][s].astype(np.float64))
    _check_expert(orc, W["sgate"].ravel(), W["sup"].ravel(), W["sdown"].ravel(),
                  shared_type, shared_type, H, Fs, xq, o["hs"].astype(np.float64), o["ys"].astype(np.float64))
    # combine: slot-weighted sum of the stored y, rounded once to bf16
    comb = (wts.astype(np.float64)[:, None] * o["y"].astype(np.float64)).sum(0)
    assert np.allclose(o["routed_exact"], comb, rtol=1e-15, atol=1e-300)
    want_bf = torch.from_numpy(o["routed_exact"].astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o["routed"], want_bf)
    sh = float(sg) * o["ys"].astype(np.float64)
    assert np.array_equal(o["shared_exact"], sh)
    want_bf = torch.from_numpy(sh.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(o["shared"], want_bf)


def test_layer_is_composition_of_steps(orc):
    cfg = wl.variant(wl.CONFIGS["layer"], E=32)           # full H/F/Fs, fewer experts for speed
    W = _np_weights(cfg)
    ti = wl.token_inputs(cfg, 0)
    pv = wl.prev_outputs(cfg, 0)
    res, rp, sp = wl.u16(ti["residual"]), wl.u16(pv["routed_prev"]), wl.u16(pv["shared_prev"])
    desc = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs)
    o = orc.moe_layer(desc, W, res, rp, sp)
    out_sum, xn, xq = orc.add_rmsnorm(res, rp, sp, W["norm_w"], cfg.eps)
    assert np.array_equal(o["out_sum"], out_sum) and np.array_equal(o["xn"], xn) and np.array_equal(o["xq"], xq)
    r = orc.router_topk(desc, W, xn)
    assert np.array_equal(o["logits"], r["logits"]) and np.array_equal(o["ids"], r["ids"])
    assert np.array_equal(o["weights"], r["weights"]) and o["shared_gate"][0] == np.float32(r["shared_gate"])
    assert np.array_equal(r["ids"], orc.topk(r["logits"], cfg.k))
    assert np.array_equal(r["weights"], orc.softmax_selected(r["logits"], r["ids"]))
    assert np.array_equal(r["logits"], orc.router(xn, W["router_w"]))
    f = orc.expert_ffn(desc, W, xq, r["ids"], r["weights"], r["shared_gate"])
    assert np.array_equal(o["routed"], f["routed"]) and np.array_equal(o["shared"], f["shared"])
    # sigmoid gate: f32(1/(1+exp(-z))) of the f32 shared-gate logit
    z = np.float32(o["z"][0])
    assert np.isclose(o["shared_gate"][0], np.float32(1.0 / (1.0 + np.exp(-np.float64(z)))), rtol=2 ** -23, atol=0)
    zw = np.dot(W["shared_gate_w"].astype(np.float64), xn.astype(np.float64))
    assert np.isclose(z, np.float32(zw), rtol=2 ** -23, atol=0)


def test_tiny_workload_ties_and_no_norm(orc):
    cfg = wl.CONFIGS["tiny"]
    W = _np_weights(cfg)
    assert np.array_equal(W["router_w"][0::2], W["router_w"][1::2])
    desc = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs, norm=0)
    for t in range(8):
        x = wl.token_inputs(cfg, t)["x"].numpy()
        o = orc.moe_layer(desc, W, x=x)
        lg = o["logits"]
        assert np.array_equal(lg[0::2], lg[1::2])                  # duplicated rows tie exactly
        ids = o["ids"]
        assert np.array_equal(ids[0::2] + 1, ids[1::2]) and np.all(ids[0::2] % 2 == 0)
        assert o["weights"][0] == o["weights"][1] and o["weights"][2] == o["weights"][3]
        assert np.array_equal(o["xq"], orc.quantize_q8_1(x)) and np.array_equal(o["xn"], x)


def test_stack_is_composition_of_layers(orc):
    cfg = wl.variant(wl.CONFIGS["layer"], E=16, layers=3)
    Ws = [_np_weights(cfg, l) for l in range(3)]
    desc = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs)
    inp = wl.u16(wl.token_inputs(cfg, 0)["residual"])
    out, per = orc.moe_stack(desc, Ws, inp, per_layer=True)
    res, rt, sh = inp, None, None
    for l in range(3):
        o = orc.moe_layer(desc, Ws[l], res, rt, sh)
        assert np.array_equal(per["ids"][l], o["ids"]) and np.array_equal(per["resid"][l], o["out_sum"])
        res, rt, sh = o["out_sum"], o["routed"], o["shared"]
    f = lambda h: (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    b = lambda v: torch.from_numpy(np.asarray(v, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    want = b(f(res) + f(b(f(rt) + f(sh))))
    assert np.array_equal(out, want)


def test_zero_token_stays_zero(orc):
    """No shared expert, no bias: an all-zero token gives 128 equal logits at every
    layer, so ids are 0..k-1 with weights 1/k, and the output stays zero."""
    cfg = wl.variant(wl.CONFIGS["e128"], H=512, E=32, F=768, layers=2)
    Ws = [_np_weights(cfg, l) for l in range(2)]
    desc = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, 0)
    out, per = orc.moe_stack(desc, Ws, np.zeros(cfg.H, np.uint16), per_layer=True)
    assert not out.any()
    assert np.all(per["ids"] == np.arange(cfg.k))
    o = orc.moe_layer(desc, Ws[0], np.zeros(cfg.H, np.uint16), None, None)
    assert np.all(o["weights"] == np.float32(1.0 / cfg.k))
    assert np.array_equal(o["routed"], np.zeros(cfg.H, np.uint16))


def test_layer_with_given_selection(orc):
    """The near-tie continuation: a layer run with a given selection.  Given
    the top-k it would pick itself, every output is bit-identical to the plain
    layer; given another selection, the routed output is the dense-pinned
    expert FFN of those experts weighted by the softmax over their own logits
    (so the rank order of the weights follows the logits, not the slots), and
    everything before the selection (norm, logits, shared gate) and the shared
    output are unchanged.  Invalid selections are refused."""
    cfg = wl.variant(wl.CONFIGS["layer"], E=32)
    W = _np_weights(cfg)
    ti, pv = wl.token_inputs(cfg, 1), wl.prev_outputs(cfg, 1)
    res, rp, sp = wl.u16(ti["residual"]), wl.u16(pv["routed_prev"]), wl.u16(pv["shared_prev"])
    desc = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs)
    o = orc.moe_layer(desc, W, res, rp, sp)
    same = orc.moe_layer(desc, W, res, rp, sp, ids=o["ids"])
    for key in ("out_sum", "xn", "xq", "logits", "ids", "weights", "shared_gate", "h", "y", "routed", "shared"):
        assert np.array_equal(o[key], same[key]), key
    # ranks k-1 and k swapped in, slot order reversed
    order = np.lexsort((np.arange(cfg.E), -o["logits"].astype(np.float64)))
    alt = np.concatenate([order[:cfg.k - 1], order[cfg.k:cfg.k + 1]])[::-1].astype(np.int32)
    a = orc.moe_layer(desc, W, res, rp, sp, ids=alt)
    assert np.array_equal(a["ids"], alt)
    for key in ("out_sum", "xn", "xq", "logits", "shared_gate", "shared"):
        assert np.array_equal(o[key], a[key]), key
    lg = o["logits"].astype(np.float64)[alt]
    p = np.exp(lg - lg[0])
    assert np.allclose(a["weights"], p / p.sum(), rtol=2 ** -22, atol=0)
    assert np.all(np.diff(a["weights"]) >= 0)          # slots go from the smallest logit up
    f = orc.expert_ffn(desc, W, o["xq"], alt, a["weights"], float(o["shared_gate"][0]))
    assert np.array_equal(a["routed"], f["routed"]) and np.array_equal(a["y"], f["y"])
    # expert alt[s]'s rows land in slot s: its y is that of the same expert in the plain run
    s_plain = {int(e): s for s, e in enumerate(o["ids"])}
    for s, e in enumerate(alt):
        if int(e) in s_plain:
            assert np.array_equal(a["y"][s], o["y"][s_plain[int(e)]])
    for bad in ([0] * cfg.k, list(range(cfg.k - 1)) + [cfg.E], list(range(cfg.k - 1)) + [-1]):
        with pytest.raises(ValueError):
            orc.moe_layer(desc, W, res, rp, sp, ids=np.array(bad, np.int32))


def test_stack_behind_attention_blocks(orc):
    """The stack with an attention block's output per layer: each layer is
    the fold of the previous outputs (u1) followed by the 2-input layer on
    (u1, attn) -- checked against that composition built from the separately
    pinned fold and layer; an all-zero attention output changes nothing
    (bf16(u1 + 0) = u1), bit for bit; and a nonzero one changes the result."""
    cfg = wl.variant(wl.CONFIGS["layer"], E=16, layers=3)
    Ws = [_np_weights(cfg, l) for l in range(3)]
    desc = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs)
    inp = wl.u16(wl.token_inputs(cfg, 0)["residual"])
    attn = np.stack([wl.u16(wl.attention_output(cfg, 0, l)) for l in range(3)])
    out, per = orc.moe_stack(desc, Ws, inp, per_layer=True, attn=attn)
    res, rt, sh = inp, None, None
    for l in range(3):
        u1 = orc.add_rmsnorm(res, rt, sh, Ws[l]["norm_w"], cfg.eps)[0] if l else res
        o = orc.moe_layer(desc, Ws[l], u1, attn[l], None)
        assert np.array_equal(per["ids"][l], o["ids"]) and np.array_equal(per["resid"][l], o["out_sum"])
        assert np.array_equal(per["routed"][l], o["routed"]) and np.array_equal(per["shared"][l], o["shared"])
        res, rt, sh = o["out_sum"], o["routed"], o["shared"]
    fin = orc.add_rmsnorm(res, rt, sh, Ws[0]["norm_w"], cfg.eps)[0]
    assert np.array_equal(out, fin)
    plain = orc.moe_stack(desc, Ws, inp)
    assert np.array_equal(orc.moe_stack(desc, Ws, inp, attn=np.zeros_like(attn)), plain)
    assert not np.array_equal(out, plain)
