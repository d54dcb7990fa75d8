"""Parity of the HIP library against the CPU oracle, element by element, on the
same seeded inputs (sizes the oracle finishes in seconds, spanning several
tiles and ragged tails), through the C ABI.

Integer and index results are compared bit for bit: sub-block dots, Q8_1
codes of identical inputs, expert ids from identical logits.  Floating-point
outputs must meet the criterion in gpu_util (bf16 = one rounding of a value
within 2e-3 of the exact result).
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
import qformats as qf
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_router_expert_amd as q
    assert torch.cuda.is_available()
    return q


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ integer dots
@pytest.mark.parametrize("typ,K", [(qf.Q4_K, 256), (qf.Q4_K, 2048), (qf.Q4_K, 768), (qf.Q5_K, 512), (qf.Q5_K, 768),
                                   (qf.Q8_0, 2048), (qf.Q8_0, 512), (qf.Q4_K, 8192)])
def test_subblock_dots_bit_exact(q, orc, typ, K):
    gu.banner(f"subblock dots type {typ} K {K}")
    n = 37
    rows = wl.quantize(wl.randn((n, K), 100 + K + typ) * 0.02, typ).numpy()
    x = np.random.default_rng(K + typ).standard_normal(K).astype(np.float32)
    x[:32] = 0.0                               # one all-zero activation block
    xq = orc.quantize_q8_1(x)
    out = torch.zeros(n, K // 32, dtype=torch.int32, device="cuda")
    q.moe_test_subblock_dots(gu.dev(rows), typ, K, n, gu.dev(xq), out)
    _sync()
    got = gu.host(out)
    for r in range(n):
        assert np.array_equal(got[r], orc.subblock_dots(rows[r], typ, K, xq)), r


# ------------------------------------------------------------------ Q8_1 quantiser of the persistent kernel
@pytest.mark.parametrize("nblk,mix", [(1000, "normal"), (1000, "mixed"), (131, "mixed"), (4096, "wide")])
def test_quantize_q81_four_lane_bit_exact(q, orc, nblk, mix):
    """The four-lane quantiser's fast operations (and its per-wave IEEE fallback
    for out-of-range maxima) give the oracle's bytes: block scales from 2^-112
    to 2^124, all-zero and one-value blocks, signed zeros."""
    gu.banner(f"four-lane Q8_1 quantiser {nblk} blocks, {mix}")
    rng = np.random.default_rng(nblk * 7 + len(mix))
    x = rng.standard_normal((nblk, 32)).astype(np.float64)
    if mix == "normal":
        e = rng.integers(-20, 21, nblk)
    elif mix == "mixed":
        e = rng.integers(-20, 21, nblk)
        far = rng.random(nblk) < 0.02            # a few blocks per wave force the fallback
        e[far] = rng.choice(np.r_[np.arange(-112, -100), np.arange(101, 125)], far.sum())
    else:
        e = rng.integers(-112, 125, nblk)
    x *= np.exp2(e)[:, None]
    kind = rng.integers(0, 12, nblk)
    x[kind == 0] = 0.0
    x[kind == 1] = -0.0
    x[kind == 2, 1:] = 0.0                       # a single nonzero value
    x = x.astype(np.float32).ravel()
    ref = orc.quantize_q8_1(x)
    out = torch.zeros(nblk * 36, dtype=torch.uint8, device="cuda")
    q.moe_test_quantize_q81(gu.dev(x), x.size, out)
    _sync()
    got = gu.host(out)
    bad = np.nonzero((got.reshape(nblk, 36) != ref.reshape(nblk, 36)).any(1))[0]
    assert bad.size == 0, f"{bad.size} blocks differ, first {bad[:5]}"


# ------------------------------------------------------------------ a1: add_rmsnorm3
@pytest.mark.parametrize("H,n_tok,form", [(2048, 1, 3), (2048, 5, 3), (2048, 3, 2), (2048, 2, 1), (512, 7, 3),
                                          (8192, 2, 3), (256, 3, 2), (2048, 4, 4), (2048, 3, 5), (512, 2, 6)])
def test_add_rmsnorm3(q, orc, H, n_tok, form):
    """form 4 = form 3 with norm weights near 1e-6: Q8_1 scales below the fp16
    range (d = 0, and s = -0 for a negative code sum).  Forms 5 and 6 = forms 3
    and 2 with every vector and the norm weight at an address that is not
    16-byte aligned (the kernel's element-wise path)."""
    gu.banner(f"add_rmsnorm3 H {H} n_tok {n_tok} form {form}")
    tiny = form == 4
    skew = form in (5, 6)
    form = 3 if form in (4, 5) else 2 if form == 6 else form
    rng = np.random.default_rng(H * 10 + n_tok + form)
    bf = lambda a: torch.from_numpy(a.astype(np.float32)).to(torch.bfloat16)
    res = bf(rng.standard_normal((n_tok, H)))
    rt = bf(rng.standard_normal((n_tok, H)) * 0.5) if form >= 2 else None
    sh = bf(rng.standard_normal((n_tok, H)) * 0.2) if form == 3 else None
    if n_tok > 2:
        res[1] = 0.0                               # an all-zero token
        if rt is not None:
            rt[1] = 0.0
        if sh is not None:
            sh[1] = 0.0
    w = torch.from_numpy(rng.uniform(0.5, 1.5, H).astype(np.float32) * (1e-6 if tiny else 1.0))
    out = torch.zeros(n_tok, H, dtype=torch.bfloat16, device="cuda")
    xn = torch.zeros(n_tok, H, dtype=torch.float32, device="cuda")
    xq = torch.zeros(n_tok, H // 32 * 36, dtype=torch.uint8, device="cuda")

    def put(t):
        # a device copy, at an address 2 (bf16) or 4 (fp32) bytes past a 16-byte boundary when skewed
        if t is None:
            return None
        if not skew:
            return t.cuda()
        flat = torch.zeros(t.numel() + 8, dtype=t.dtype, device="cuda")
        flat[1:1 + t.numel()] = t.reshape(-1).cuda()
        return flat[1:1 + t.numel()].view(t.shape)

    if skew:
        out_s, xn_s = put(out), put(xn)
        q.add_rmsnorm3(put(res), put(rt), put(sh), put(w), H, n_tok, 1e-6, out_s, xn_s, xq)
        _sync()
        out.copy_(out_s)
        xn.copy_(xn_s)
    else:
        q.add_rmsnorm3(put(res), put(rt), put(sh), put(w), H, n_tok, 1e-6, out, xn, xq)
    _sync()
    g_out, g_xn, g_xq = gu.u16_host(out), gu.host(xn), gu.host(xq)
    for t in range(n_tok):
        o_out, o_xn, o_xq = orc.add_rmsnorm(wl.u16(res[t]), wl.u16(rt[t]) if rt is not None else None,
                                            wl.u16(sh[t]) if sh is not None else None, w.numpy(), 1e-6)
        assert np.array_equal(g_out[t], o_out), t               # pure bf16 adds: bit-exact
        gu.assert_f32_within(g_xn[t], o_xn, f"xn tok {t}")
        # xn is computed in fp64 with one rounding: it matches the oracle except within an
        # fp64 ulp of an fp32 rounding boundary (the sum of squares is reduced in another order)
        d = gu.ulp_diff_f32(g_xn[t], o_xn)
        assert d.max() <= 1 and (d > 0).sum() <= 1, (d.max(), (d > 0).sum())
        same_blocks = (g_xn[t].reshape(-1, 32) == o_xn.reshape(-1, 32)).all(1)
        gb, ob = g_xq[t].reshape(-1, 36), o_xq.reshape(-1, 36)
        assert np.array_equal(gb[same_blocks], ob[same_blocks])  # identical inputs -> identical Q8_1 bytes


# ------------------------------------------------------------------ a2+a3 from identical logits
def _identity_router(E, H):
    W = np.zeros((E, H), np.float32)
    W[np.arange(E), np.arange(E)] = 1.0
    return W


@pytest.mark.parametrize("E,k", [(256, 8), (32, 4), (128, 8), (1024, 16), (8, 8), (64, 1)])
def test_topk_identical_logits_tie_heavy(q, orc, E, k):
    """W = identity makes the GPU's logits exactly the given values, so the selection
    is compared from identical logits: 4000 tie-heavy sets per shape."""
    gu.banner(f"topk tie-heavy E {E} k {k}")
    H = max(256, (E + 255) // 256 * 256)
    n = 4000
    rng = np.random.default_rng(E * 100 + k)
    L = np.zeros((n, H), np.float32)
    for t in range(n):
        levels = rng.standard_normal(int(rng.integers(1, 6))).astype(np.float32)
        L[t, :E] = levels[rng.integers(0, levels.size, E)]
        if t % 5 == 0:
            L[t, rng.integers(0, E, 3)] = rng.standard_normal(3).astype(np.float32)
        if t % 97 == 0:
            L[t, :E] = 0.0                         # all equal
        if t % 89 == 0:
            L[t, :E] = np.repeat(rng.standard_normal(E // 2 if E > 1 else 1).astype(np.float32), 2)[:E]
    W = _identity_router(E, H)
    ids = torch.zeros(n, k, dtype=torch.int32, device="cuda")
    wts = torch.zeros(n, k, dtype=torch.float32, device="cuda")
    lg = torch.zeros(n, E, dtype=torch.float32, device="cuda")
    ws = torch.zeros(q.router_ws_bytes(n, E) + 256, dtype=torch.uint8, device="cuda")
    ws = ws[(-ws.data_ptr()) % 256:][:q.router_ws_bytes(n, E)]
    q.moe_workspace_init(ws)
    q.router_topk(gu.dev(L), gu.dev(W), None, n, H, E, k, lg, ids, wts, None, ws)
    _sync()
    g_ids, g_w, g_lg = gu.host(ids), gu.host(wts), gu.host(lg)
    assert np.array_equal(g_lg, L[:, :E])
    for t in range(n):
        o_ids = orc.topk(L[t, :E], k)
        assert np.array_equal(g_ids[t], o_ids), t
        gu.assert_f32_within(g_w[t], orc.softmax_selected(L[t, :E], o_ids), f"weights tok {t}")
    # the handshake counter wrapped back to zero: a second launch behaves the same
    ids2 = torch.zeros_like(ids)
    q.router_topk(gu.dev(L), gu.dev(W), None, n, H, E, k, None, ids2, wts, None, ws)
    _sync()
    assert torch.equal(ids, ids2)
    assert int(ws[:4 * n].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("n", [1, 8, 112, 113, 1024, 1025])
def test_router_counter_layouts(q, orc, n):
    """The last-workgroup handshake in each of its counter layouts: eight
    sub-counters and a top counter per token group (up to 14 groups of 8
    tokens), one counter per 128-byte line (up to 128 groups), one per word
    beyond.  Selection from identical logits (identity router) must match
    the oracle on every token, twice in a row, and every counter word must be
    back at zero after each launch."""
    E, k, H = 256, 8, 256
    gu.banner(f"router counter layouts n {n}")
    rng = np.random.default_rng(n)
    L = np.zeros((n, H), np.float32)
    L[:, :E] = rng.standard_normal((n, E)).astype(np.float32)
    L[::7, :E] = np.round(L[::7, :E])             # some tie-heavy tokens
    W = _identity_router(E, H)
    nb = q.router_ws_bytes(n, E)
    ws = torch.zeros(nb + 256, dtype=torch.uint8, device="cuda")
    ws = ws[(-ws.data_ptr()) % 256:][:nb]
    q.moe_workspace_init(ws)
    counter_bytes = 4 * 4096                      # the counter area ahead of the logits
    ref = np.stack([orc.topk(L[t, :E], k) for t in range(n)])
    for rep in range(2):
        ids = torch.full((n, k), -1, dtype=torch.int32, device="cuda")
        wts = torch.zeros(n, k, dtype=torch.float32, device="cuda")
        q.router_topk(gu.dev(L), gu.dev(W), None, n, H, E, k, None, ids, wts, None, ws)
        _sync()
        assert np.array_equal(gu.host(ids), ref), rep
        assert int(ws[:counter_bytes].view(torch.int32).abs().sum()) == 0, rep


@pytest.mark.parametrize("cfg_name", ["tiny", "layer", "e128"])
def test_router_topk_real(q, orc, cfg_name):
    cfg = wl.CONFIGS[cfg_name]
    gu.banner(f"router_topk {cfg_name}")
    E, H, k = cfg.E, cfg.H, cfg.k
    Wr = wl._router_rows(cfg, 0, "cpu").numpy()
    g = wl.randn((H,), 77, "cpu", cfg.weight_std).numpy() if cfg.Fs > 0 else None
    n = 64
    X = np.random.default_rng(5).standard_normal((n, H)).astype(np.float32)
    X[3] = 0.0
    ids = torch.zeros(n, k, dtype=torch.int32, device="cuda")
    wts = torch.zeros(n, k, dtype=torch.float32, device="cuda")
    lg = torch.zeros(n, E, dtype=torch.float32, device="cuda")
    sg = torch.zeros(n, dtype=torch.float32, device="cuda")
    nb = q.router_ws_bytes(n, E)
    ws = torch.zeros(nb + 256, dtype=torch.uint8, device="cuda")
    ws = ws[(-ws.data_ptr()) % 256:][:nb]
    q.moe_workspace_init(ws)
    q.router_topk(gu.dev(X), gu.dev(Wr), gu.dev(g) if g is not None else None, n, H, E, k, lg, ids, wts,
                  sg if g is not None else None, ws)
    _sync()
    g_lg, g_ids, g_w, g_sg = gu.host(lg), gu.host(ids), gu.host(wts), gu.host(sg)
    desc = orc.make_desc(H, E, k, cfg.F, cfg.Fs)
    W = {"router_w": Wr, "shared_gate_w": g}
    exact_lg = 0
    for t in range(n):
        o = orc.router_topk(desc, W, X[t])
        d = gu.ulp_diff_f32(g_lg[t], o["logits"])
        assert d.max() <= 1, d.max()            # fp64 sums of exact products, one rounding each
        exact_lg += int((d == 0).all())
        if np.array_equal(g_lg[t], o["logits"]):
            assert np.array_equal(g_ids[t], o["ids"]), t
            gu.assert_f32_within(g_w[t], o["weights"], f"weights {t}")
        if g is not None:
            gu.assert_f32_within(g_sg[t:t + 1], [o["shared_gate"]], f"sigmoid gate {t}")
        if cfg.router_dup > 1:                  # duplicated rows tie exactly on the GPU too
            r = g_lg[t].reshape(-1, cfg.router_dup)
            assert (r == r[:, :1]).all()
    assert exact_lg >= n - 2
    assert np.array_equal(g_ids[3], np.arange(k))   # zero input: all logits equal


# ------------------------------------------------------------------ a4+a5+a6: expert FFN, stage-isolated
FFN_CASES = [("tiny", wl.Q4_K, wl.Q4_K), ("layer", wl.Q4_K, wl.Q4_K), ("layer", wl.Q8_0, wl.Q5_K), ("e128", wl.Q4_K, wl.Q4_K)]


def _gpu_weights(cfg, layer, shared_type, down_type):
    w = wl.layer_weights(cfg, layer, "cuda", shared_type=shared_type, down_type=down_type)
    return w, wl.to_numpy_weights(w)


@pytest.mark.parametrize("cfg_name,shared_type,down_type", FFN_CASES)
def test_expert_ffn_stage_isolated(q, orc, cfg_name, shared_type, down_type):
    cfg = wl.CONFIGS[cfg_name]
    gu.banner(f"expert_ffn {cfg_name} shared {shared_type} down {down_type}")
    W, Wn = _gpu_weights(cfg, 0, shared_type, down_type)
    H, F, Fs, k, E = cfg.H, cfg.F, cfg.Fs, cfg.k, cfg.E
    desc_o = orc.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, norm=0)
    desc_g = q.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, norm=0)
    ws = q.alloc_workspace(desc_g)
    rng = np.random.default_rng(H + F)
    for trial in range(3):
        x = rng.standard_normal(H).astype(np.float32)
        xq = orc.quantize_q8_1(x)
        ids = rng.choice(E, size=k, replace=False).astype(np.int32)
        if trial == 1:
            ids[:] = np.arange(E - k, E)                 # the last experts (end of the stacked matrices)
        lgt = rng.standard_normal(k).astype(np.float32)
        wts = np.sort(np.exp(lgt) / np.exp(lgt).sum()).astype(np.float32)[::-1].copy()
        sgv = np.float32(rng.uniform(0.05, 0.95))
        routed = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
        shared = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
        h = torch.zeros(k, F, dtype=torch.float32, device="cuda")
        hs = torch.zeros(max(Fs, 1), dtype=torch.float32, device="cuda")
        q.expert_ffn_q4k(desc_g, W, gu.dev(xq), gu.dev(ids), gu.dev(wts), gu.dev(np.array([sgv])), 1, routed,
                         shared if Fs > 0 else None, h, hs if Fs > 0 else None, ws)
        _sync()
        o = orc.expert_ffn(desc_o, Wn, xq, ids, wts, float(sgv))
        gh = gu.host(h)
        gu.assert_f32_within(gh, o["h"], "h")
        dh = gu.ulp_diff_f32(gh, o["h"])
        assert (dh > 0).mean() < 1e-3, (dh > 0).sum()      # one fp32 rounding of an fp64 row sum each
        gu.assert_bf16_within(gu.u16_host(routed), o["routed_exact"], "routed")
        if Fs > 0:
            gu.assert_f32_within(gu.host(hs)[:Fs], o["hs"], "hs")
            gu.assert_bf16_within(gu.u16_host(shared), o["shared_exact"], "shared")
        print(f"  trial {trial}: h exact {float((dh == 0).mean()):.5f} routed exact "
              f"{float((gu.u16_host(routed) == o['routed']).mean()):.5f}", flush=True)


# ------------------------------------------------------------------ a1..a6: whole layer, chained
# wide expert sets for the gate/up kernel's selection: more than 256 experts
# (picks by wave-wide maxima in the four selecting waves) and top-k above 8
# (16 candidate slots per wave), with duplicated router rows for ties
WIDE = {"wide320": wl.Config("wide320", H=512, E=320, k=12, F=128, Fs=128, router_dup=2, config_index=11),
        "wide1024": wl.Config("wide1024", H=512, E=1024, k=16, F=128, Fs=0, three_input=False, router_dup=4,
                              config_index=12)}
LAYER_CASES = [("tiny", wl.Q4_K, wl.Q4_K, 8), ("layer", wl.Q4_K, wl.Q4_K, 4), ("layer", wl.Q8_0, wl.Q5_K, 2),
               ("e128", wl.Q4_K, wl.Q4_K, 3), ("wide320", wl.Q4_K, wl.Q4_K, 3), ("wide1024", wl.Q4_K, wl.Q4_K, 2)]


@pytest.mark.parametrize("cfg_name,shared_type,down_type,ntok", LAYER_CASES)
def test_decode_layer_chained(q, orc, cfg_name, shared_type, down_type, ntok):
    cfg = WIDE.get(cfg_name) or wl.CONFIGS[cfg_name]
    gu.banner(f"moe_decode_layer {cfg_name} shared {shared_type} down {down_type}")
    W, Wn = _gpu_weights(cfg, 0, shared_type, down_type)
    H, F, Fs, k, E = cfg.H, cfg.F, cfg.Fs, cfg.k, cfg.E
    norm = 1 if cfg.norm else 0
    desc_o = orc.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, norm=norm, eps=cfg.eps)
    desc_g = q.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, norm=norm, eps=cfg.eps)
    ws = q.alloc_workspace(desc_g)
    for t in range(ntok):
        ti = wl.token_inputs(cfg, t, "cpu")
        io = {"routed_out": torch.zeros(H, dtype=torch.bfloat16, device="cuda"),
              "xn": torch.zeros(H, dtype=torch.float32, device="cuda"),
              "xq": torch.zeros(H // 32 * 36, dtype=torch.uint8, device="cuda"),
              "logits": torch.zeros(E, dtype=torch.float32, device="cuda"),
              "ids": torch.zeros(k, dtype=torch.int32, device="cuda"),
              "weights": torch.zeros(k, dtype=torch.float32, device="cuda"),
              "h": torch.zeros(k, F, dtype=torch.float32, device="cuda")}
        if Fs > 0:
            io["shared_out"] = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
            io["shared_gate"] = torch.zeros(1, dtype=torch.float32, device="cuda")
            io["hs"] = torch.zeros(Fs, dtype=torch.float32, device="cuda")
        if norm:
            pv = wl.prev_outputs(cfg, t, "cpu")
            if t == ntok - 1 and cfg_name == "e128":
                ti["residual"] = torch.zeros_like(ti["residual"])       # a zero token
                pv = {"routed_prev": torch.zeros_like(pv["routed_prev"])}
            io["residual"] = ti["residual"].cuda()
            io["routed_in"] = pv["routed_prev"].cuda()
            io["shared_in"] = pv["shared_prev"].cuda() if "shared_prev" in pv else None
            io["out_sum"] = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
            o = orc.moe_layer(desc_o, Wn, wl.u16(ti["residual"]), wl.u16(pv["routed_prev"]),
                              wl.u16(pv["shared_prev"]) if "shared_prev" in pv else None)
        else:
            io["x"] = ti["x"].cuda()
            o = orc.moe_layer(desc_o, Wn, x=ti["x"].numpy())
        q.moe_decode_layer(desc_g, W, io, ws)
        _sync()
        if norm:
            assert np.array_equal(gu.u16_host(io["out_sum"]), o["out_sum"])
        g_xn = gu.host(io["xn"])
        assert gu.ulp_diff_f32(g_xn, o["xn"]).max() <= 1
        same_blocks = (g_xn.reshape(-1, 32) == o["xn"].reshape(-1, 32)).all(1)
        gb, ob = gu.host(io["xq"]).reshape(-1, 36), o["xq"].reshape(-1, 36)
        assert np.array_equal(gb[same_blocks], ob[same_blocks])  # identical inputs -> identical Q8_1 bytes
        assert gu.ulp_diff_f32(gu.host(io["logits"]), o["logits"]).max() <= 1
        same_logits = np.array_equal(gu.host(io["logits"]), o["logits"])
        g_ids = gu.host(io["ids"])
        if same_logits:
            assert np.array_equal(g_ids, o["ids"])
        else:
            # logits differ in the last bit somewhere: the selection must still be valid
            # for the oracle's logits up to that difference
            lo = o["logits"].astype(np.float64)
            kth = np.sort(lo)[::-1][k - 1]
            assert np.all(lo[g_ids] >= kth - 4 * np.spacing(np.float32(abs(kth)))), (g_ids, o["ids"])
            if not np.array_equal(g_ids, o["ids"]):
                # the near-tie continuation: the oracle takes the GPU's selection
                print(f"  token {t}: near-tie selection differs; oracle continues with the GPU's", flush=True)
                if norm:
                    o = orc.moe_layer(desc_o, Wn, wl.u16(ti["residual"]), wl.u16(pv["routed_prev"]),
                                      wl.u16(pv["shared_prev"]) if "shared_prev" in pv else None, ids=g_ids)
                else:
                    o = orc.moe_layer(desc_o, Wn, x=ti["x"].numpy(), ids=g_ids)
        gu.assert_f32_within(gu.host(io["weights"]), o["weights"], "weights")
        gu.assert_bf16_within(gu.u16_host(io["routed_out"]), o["routed_exact"], "routed")
        if Fs > 0:
            gu.assert_bf16_within(gu.u16_host(io["shared_out"]), o["shared_exact"], "shared")
        print(f"  token {t}: ids {g_ids.tolist()} routed exact "
              f"{float((gu.u16_host(io['routed_out']) == o['routed']).mean()):.5f}", flush=True)
        if norm:
            # the residual updated in place (out_sum is the residual buffer): same results
            io2 = {n: (v.clone() if isinstance(v, torch.Tensor) else v) for n, v in io.items()}
            io2["out_sum"] = io2["residual"]
            for n in ("routed_out", "shared_out", "ids", "weights"):
                if n in io2:
                    io2[n].zero_()
            q.moe_decode_layer(desc_g, W, io2, ws)
            _sync()
            assert np.array_equal(gu.u16_host(io2["residual"]), gu.u16_host(io["out_sum"]))
            for n in ("routed_out", "shared_out", "ids", "weights"):
                if n in io2:
                    assert torch.equal(io2[n], io[n]), n


# ------------------------------------------------------------------ a7: stack, per-layer kernels
@pytest.mark.parametrize("cfg_name,L,E,st,dt,attn", [("stack", 40, 256, wl.Q4_K, wl.Q4_K, False),
                                                    ("stack", 6, 256, wl.Q8_0, wl.Q5_K, False),
                                                    ("e128", 8, 128, wl.Q4_K, wl.Q4_K, False),
                                                    ("stack", 6, 256, wl.Q4_K, wl.Q4_K, True),
                                                    ("e128", 4, 128, wl.Q4_K, wl.Q4_K, True)])
def test_stack_kernels_mode(q, orc, cfg_name, L, E, st, dt, attn):
    """The stack on the per-layer kernels (four launches per layer, one more
    behind an attention block, and the final fold), with the per-layer
    stage-isolated and chained checks."""
    import stack_check as sc
    cfg = wl.variant(wl.CONFIGS[cfg_name], layers=L, E=E)
    gu.banner(f"moe_decode_stack kernels {cfg_name} L {L} shared {st} down {dt} attention {attn}")
    sc.run_and_check(q, orc, cfg, st, dt, [0, 1], q.MOE_STACK_KERNELS, with_attn=attn)
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ determinism and graph replays
def test_layer_deterministic_and_1000_graph_replays(q, orc):
    cfg = wl.CONFIGS["layer"]
    gu.banner("determinism + graph replay")
    W, _ = _gpu_weights(cfg, 0, wl.Q4_K, wl.Q4_K)
    H, k = cfg.H, cfg.k
    desc_g = q.make_desc(H, cfg.E, k, cfg.F, cfg.Fs)
    ws = q.alloc_workspace(desc_g)
    ti, pv = wl.token_inputs(cfg, 0, "cuda"), wl.prev_outputs(cfg, 0, "cuda")
    io = {"residual": ti["residual"], "routed_in": pv["routed_prev"], "shared_in": pv["shared_prev"],
          "out_sum": torch.zeros(H, dtype=torch.bfloat16, device="cuda"),
          "routed_out": torch.zeros(H, dtype=torch.bfloat16, device="cuda"),
          "shared_out": torch.zeros(H, dtype=torch.bfloat16, device="cuda"),
          "ids": torch.zeros(k, dtype=torch.int32, device="cuda")}
    q.moe_decode_layer(desc_g, W, io, ws)
    _sync()
    ref = {n: io[n].clone() for n in ("out_sum", "routed_out", "shared_out", "ids")}
    for _ in range(100):
        q.moe_decode_layer(desc_g, W, io, ws)
    _sync()
    for n in ref:
        assert torch.equal(io[n], ref[n]), n
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q.moe_decode_layer(desc_g, W, io, ws)          # warm-up on the capture stream
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q.moe_decode_layer(desc_g, W, io, ws)
    # 1000 replays, each checked, with eager work of the program between every
    # tenth; stops at the first mismatch; the router's handshake counters are
    # back at zero after every check (no reset node is ever recorded)
    cnt = ws[:16384].view(torch.int32)
    for rep in range(1000):
        for n in ("routed_out", "shared_out", "out_sum"):
            io[n].zero_()
        io["ids"].fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(io[n], ref[n]), (rep, n)
        assert int(cnt.abs().sum()) == 0, rep
        if rep % 10 == 9:
            q.moe_decode_layer(desc_g, W, io, ws)      # eager work between replays
            torch.cuda.synchronize()


@pytest.mark.parametrize("n_tok", [1, 5])
def test_add_rmsnorm2_q8(q, orc, n_tok):
    """The post-attention add-norm: out_sum bit-exact, xn within one fp32 ulp,
    Q8_1 bytes identical wherever the xn block is identical."""
    cfg = wl.CONFIGS["layer"]
    H = cfg.H
    gu.banner(f"add_rmsnorm2_q8 n_tok {n_tok}")
    w = wl.rand_uniform((H,), 5, 0.5, 1.5)
    res = torch.stack([wl.token_inputs(cfg, t)["residual"] for t in range(n_tok)])
    att = torch.stack([wl.attention_output(cfg, t, 0) for t in range(n_tok)])
    out = torch.zeros(n_tok, H, dtype=torch.bfloat16, device="cuda")
    xn = torch.zeros(n_tok, H, dtype=torch.float32, device="cuda")
    xq = torch.zeros(n_tok, H // 32 * 36, dtype=torch.uint8, device="cuda")
    q.add_rmsnorm2_q8(res.cuda(), att.cuda(), w.cuda(), H, n_tok, cfg.eps, out, xn, xq)
    torch.cuda.synchronize()
    for t in range(n_tok):
        o_out, o_xn, o_xq = orc.add_rmsnorm(wl.u16(res[t]), wl.u16(att[t]), None, w.numpy(), cfg.eps)
        assert np.array_equal(gu.u16_host(out)[t], o_out)
        d = gu.ulp_diff_f32(gu.host(xn)[t], o_xn)
        assert d.max() <= 1
        same = (gu.host(xn)[t].reshape(-1, 32) == o_xn.reshape(-1, 32)).all(1)
        assert np.array_equal(gu.host(xq)[t].reshape(-1, 36)[same], o_xq.reshape(-1, 36)[same])
