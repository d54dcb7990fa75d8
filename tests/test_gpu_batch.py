"""Parity of the grouped batch path (several tokens, experts grouped) against
the oracle.

Groups of group_min or more tokens run on the int8 matrix cores and give each
token the value of the single-token integer path (the same integer sub-block
dots, the same fp64 task expression, the same summation tree), smaller
groups run that path member by member: the grouped path is batch-invariant.
Its reference is the oracle's grouped definition, which the oracle's own
tests pin to its single-token path.

Stage-isolated: the oracle's own xn, Q8_1 xq, ids, weights and gates go into
expert_ffn_grouped; every h must match the oracle's fp32 value to one
rounding, and the bf16 outputs must meet the 2e-3 bar against the oracle's
unrounded values.  Batch invariance: the grouped outputs (h and the bf16
routed and shared vectors) equal, bit for bit, those of the single-token call
expert_ffn_q4k run per token on the same inputs, at group_min 1 (every group
on the matrix cores) and 4.  Chained: moe_decode_layer_batch from the raw
inputs must pick the oracle's experts, match out_sum bit for bit, and keep
routed and shared within a relative L2 distance of 2e-3 per token of the
oracle's bf16 outputs.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_router_expert_amd as q
    assert torch.cuda.is_available()
    return q


SMALL = wl.Config("small", H=512, E=16, k=4, F=128, Fs=256, router_dup=2, config_index=9)
# more than 256 experts and top-12: the router's one-wave selection with eight
# keys per lane, and groups built from twelve slots per token
WIDE = wl.Config("wide", H=512, E=320, k=12, F=128, Fs=128, router_dup=2, config_index=13)


def _inputs(cfg, n):
    if cfg.config_index == 4:
        inp, _, _ = wl.batch_inputs(cfg, n)
        return {k: wl.u16(v) for k, v in inp.items()}
    res = torch.stack([wl.randn((cfg.H,), wl.seed_for(cfg.config_index, 0, wl.T_INPUT, t)) for t in range(n)])
    rp = torch.stack([wl.randn((cfg.H,), wl.seed_for(cfg.config_index, 0, wl.T_RPREV, t)) for t in range(n)])
    sp = torch.stack([wl.randn((cfg.H,), wl.seed_for(cfg.config_index, 0, wl.T_SPREV, t)) for t in range(n)])
    return {"residual": wl.u16(res.to(torch.bfloat16)), "routed_prev": wl.u16(rp.to(torch.bfloat16)),
            "shared_prev": wl.u16(sp.to(torch.bfloat16))}


_WEIGHTS = {}


def _weights(cfg, shared_type, down_type):
    key = (cfg.name, shared_type, down_type)
    if key not in _WEIGHTS:
        _WEIGHTS.clear()
        w = wl.layer_weights(cfg, 0, "cuda", shared_type=shared_type, down_type=down_type)
        _WEIGHTS[key] = (w, wl.to_numpy_weights(w))
    return _WEIGHTS[key]


CASES = [
    # (config, n_tok, group_min, shared type, down type)
    ("batch", 8, 4, wl.Q4_K, wl.Q4_K),
    ("batch", 32, 4, wl.Q4_K, wl.Q4_K),
    ("batch", 32, 1, wl.Q4_K, wl.Q4_K),      # every group on the matrix cores
    ("batch", 32, 16, wl.Q8_0, wl.Q5_K),     # shared Q8_0 + down Q5_K, nearly all groups integer
    ("small", 6, 2, wl.Q8_0, wl.Q5_K),       # K < 256 padding of the down rows (F = 128 -> 256)
    ("small", 64, 3, wl.Q4_K, wl.Q4_K),      # the largest batch: 4 column tiles
]


def _cfg(name):
    return {"small": SMALL, "wide": WIDE}.get(name) or wl.CONFIGS[name]


@pytest.mark.parametrize("cfg_name,n,gmin,shared_type,down_type", CASES)
def test_grouped_ffn_stage_isolated(q, orc, cfg_name, n, gmin, shared_type, down_type):
    cfg = _cfg(cfg_name)
    gu.banner(f"grouped ffn {cfg_name} n {n} group_min {gmin} shared {shared_type} down {down_type}")
    W, Wn = _weights(cfg, shared_type, down_type)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_o = orc.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, eps=cfg.eps)
    d_g = q.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, eps=cfg.eps)
    inp = _inputs(cfg, n)
    o = orc.moe_layer_batch(d_o, Wn, n, **inp)
    ws = q.alloc_batch_workspace(d_g, n)
    routed = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    shared = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    h = torch.zeros(n, k, F, dtype=torch.float32, device="cuda")
    hs = torch.zeros(n, Fs, dtype=torch.float32, device="cuda")
    q.expert_ffn_grouped(d_g, W, gu.dev(o["xn"]), gu.dev(o["xq"]), gu.dev(o["ids"]), gu.dev(o["weights"]),
                         gu.dev(o["shared_gate"]), n, gmin, routed, shared, h, hs, ws)
    torch.cuda.synchronize()
    gh, ghs = gu.host(h), gu.host(hs)
    for what, g, r in (("h", gh, o["h"]), ("hs", ghs, o["hs"])):
        gu.assert_f32_within(g, r, what)
        dh = gu.ulp_diff_f32(g, r)
        assert dh.max() <= 1 and (dh > 0).mean() < 1e-3, (what, int((dh > 0).sum()), int(dh.max()))
    routed_exact = np.einsum("ts,tsh->th", o["weights"].astype(np.float64), o["y"].astype(np.float64))
    shared_exact = o["shared_gate"].astype(np.float64)[:, None] * o["ys"].astype(np.float64)
    gu.assert_bf16_within(gu.u16_host(routed), routed_exact, "routed")
    gu.assert_bf16_within(gu.u16_host(shared), shared_exact, "shared")
    big = o["group_size"] >= gmin
    print(f"  groups >= {gmin} (matrix cores): {int(big.sum())} of {big.size} slots; h exact "
          f"{float((gh == o['h']).mean()):.5f}; routed exact "
          f"{float((gu.u16_host(routed) == o['routed']).mean()):.5f}, shared exact "
          f"{float((gu.u16_host(shared) == o['shared']).mean()):.5f}", flush=True)


@pytest.mark.parametrize("cfg_name,n,gmin,shared_type,down_type",
                         [("batch", 32, 1, wl.Q4_K, wl.Q4_K), ("batch", 32, 4, wl.Q4_K, wl.Q4_K),
                          ("batch", 8, 2, wl.Q8_0, wl.Q5_K), ("small", 40, 3, wl.Q4_K, wl.Q4_K)])
def test_grouped_is_batch_invariant(q, orc, cfg_name, n, gmin, shared_type, down_type):
    cfg = _cfg(cfg_name)
    gu.banner(f"grouped = single-token, bit for bit: {cfg_name} n {n} group_min {gmin} shared {shared_type} "
              f"down {down_type}")
    W, Wn = _weights(cfg, shared_type, down_type)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_o = orc.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, eps=cfg.eps)
    d_g = q.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, eps=cfg.eps)
    o = orc.moe_layer_batch(d_o, Wn, n, **_inputs(cfg, n))
    xq, ids, wts, sg = gu.dev(o["xq"]), gu.dev(o["ids"]), gu.dev(o["weights"]), gu.dev(o["shared_gate"])
    ws = q.alloc_batch_workspace(d_g, n)
    routed = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    shared = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    h = torch.zeros(n, k, F, dtype=torch.float32, device="cuda")
    hs = torch.zeros(n, Fs, dtype=torch.float32, device="cuda")
    q.expert_ffn_grouped(d_g, W, gu.dev(o["xn"]), xq, ids, wts, sg, n, gmin, routed, shared, h, hs, ws)
    ws1 = q.alloc_workspace(d_g)
    routed1 = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    shared1 = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    h1 = torch.zeros(n, k, F, dtype=torch.float32, device="cuda")
    hs1 = torch.zeros(n, Fs, dtype=torch.float32, device="cuda")
    for t in range(n):
        q.expert_ffn_q4k(d_g, W, xq[t], ids[t], wts[t], sg[t:t + 1], 1, routed1[t], shared1[t], h1[t], hs1[t], ws1)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int32), h1.view(torch.int32))
    assert torch.equal(hs.view(torch.int32), hs1.view(torch.int32))
    assert torch.equal(routed.view(torch.int16), routed1.view(torch.int16))
    assert torch.equal(shared.view(torch.int16), shared1.view(torch.int16))
    big = o["group_size"] >= gmin
    print(f"  {int(big.sum())} of {big.size} slots on the matrix cores; all outputs bit-identical", flush=True)


@pytest.mark.parametrize("cfg_name,n,gmin", [("batch", 8, 4), ("batch", 32, 4), ("small", 12, 3), ("wide", 24, 3)])
def test_decode_layer_batch_chained(q, orc, cfg_name, n, gmin):
    cfg = _cfg(cfg_name)
    gu.banner(f"decode_layer_batch {cfg_name} n {n} group_min {gmin}")
    W, Wn = _weights(cfg, wl.Q4_K, wl.Q4_K)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_o = orc.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    d_g = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    inp = _inputs(cfg, n)
    o = orc.moe_layer_batch(d_o, Wn, n, **inp)
    ws = q.alloc_batch_workspace(d_g, n)
    io = {"residual": gu.dev_u16(inp["residual"]), "routed_in": gu.dev_u16(inp["routed_prev"]),
          "shared_in": gu.dev_u16(inp["shared_prev"]),
          "out_sum": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
          "routed_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
          "shared_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
          "ids": torch.zeros(n, k, dtype=torch.int32, device="cuda"),
          "weights": torch.zeros(n, k, dtype=torch.float32, device="cuda")}
    q.moe_decode_layer_batch(d_g, W, io, n, gmin, ws)
    torch.cuda.synchronize()
    assert np.array_equal(gu.u16_host(io["out_sum"]), o["out_sum"])
    assert np.array_equal(gu.host(io["ids"]), o["ids"])
    gu.assert_f32_within(gu.host(io["weights"]), o["weights"], "weights")
    worst = 0.0
    # bf16 outputs against the oracle's bf16 outputs: the rounding of the outputs
    # themselves (up to 2^-9 relative) is common to both and not an error
    for key, ref in (("routed_out", o["routed"]), ("shared_out", o["shared"])):
        g = gu.bf16_bits_to_f64(gu.u16_host(io[key]))
        r = gu.bf16_bits_to_f64(ref)
        rel = np.linalg.norm(g - r, axis=1) / np.linalg.norm(r, axis=1)
        assert rel.max() <= 2e-3, (key, rel.max())
        worst = max(worst, float(rel.max()))
    print(f"  worst per-token relative L2 error {worst:.2e}; routed exact "
          f"{float((gu.u16_host(io['routed_out']) == o['routed']).mean()):.5f}", flush=True)


def test_grouped_ffn_bad_ids_give_nan(q, orc):
    cfg = SMALL
    gu.banner("grouped ffn: an id out of range")
    W, Wn = _weights(cfg, wl.Q4_K, wl.Q4_K)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_g = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    n = 4
    ws = q.alloc_batch_workspace(d_g, n)
    xn = torch.randn(n, H, device="cuda")
    xq = torch.zeros(n, H // 32 * 36, dtype=torch.uint8, device="cuda")
    ids = torch.arange(n * k, dtype=torch.int32, device="cuda").reshape(n, k) % E
    ids[2, 1] = E + 5
    wts = torch.full((n, k), 1.0 / k, device="cuda")
    sg = torch.full((n,), 0.5, device="cuda")
    routed = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    shared = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    q.expert_ffn_grouped(d_g, W, xn, xq, ids, wts, sg, n, 2, routed, shared, None, None, ws)
    torch.cuda.synchronize()
    assert torch.isnan(routed.float()).all() and torch.isnan(shared.float()).all()


def test_decode_layer_batch_graph_replays(q, orc):
    """The matrix-core groups run on a second stream forked from the caller's
    and joined before the combine: a call captured into a HIP graph (after an
    eager call, so the fork is in the graph) must give the eager call's
    outputs bit for bit on every replay, with other work between replays."""
    cfg = wl.CONFIGS["batch"]
    n, gmin = 32, 4
    gu.banner(f"decode_layer_batch in a graph: batch {n} group_min {gmin}, 5 replays")
    W, _ = _weights(cfg, wl.Q4_K, wl.Q4_K)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_g = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    inp = _inputs(cfg, n)
    ws = q.alloc_batch_workspace(d_g, n)

    def io_new():
        return {"residual": gu.dev_u16(inp["residual"]), "routed_in": gu.dev_u16(inp["routed_prev"]),
                "shared_in": gu.dev_u16(inp["shared_prev"]),
                "out_sum": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "routed_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "shared_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "ids": torch.zeros(n, k, dtype=torch.int32, device="cuda")}

    ref = io_new()
    q.moe_decode_layer_batch(d_g, W, ref, n, gmin, ws)
    torch.cuda.synchronize()
    io = io_new()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        q.moe_decode_layer_batch(d_g, W, io, n, gmin, ws)
    torch.cuda.synchronize()
    for r in range(5):
        for key in ("out_sum", "routed_out", "shared_out"):
            io[key].fill_(float("nan"))
        io["ids"].fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for key in ("out_sum", "routed_out", "shared_out"):
            assert torch.equal(io[key].view(torch.int16), ref[key].view(torch.int16)), (r, key)
        assert torch.equal(io["ids"], ref["ids"]), r
        # eager work between replays: the same call on other buffers
        other = io_new()
        q.moe_decode_layer_batch(d_g, W, other, n, gmin, ws)
        torch.cuda.synchronize()
        assert torch.equal(other["routed_out"].view(torch.int16), ref["routed_out"].view(torch.int16)), r
    print("  5 replays bit-identical to the eager call", flush=True)


def test_decode_layer_batch_two_threads(q, orc):
    """Two host threads, each on its own stream and workspace, calling the
    batch path at once (both with matrix-core and integer-path groups, so both
    fork onto the device's shared second stream): every call's outputs equal
    a single-threaded call's bit for bit."""
    import threading
    cfg = wl.CONFIGS["batch"]
    n, gmin = 32, 4
    gu.banner(f"decode_layer_batch from two host threads: batch {n} group_min {gmin}, 10 calls each")
    W, _ = _weights(cfg, wl.Q4_K, wl.Q4_K)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_g = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    inp = _inputs(cfg, n)

    def io_new():
        return {"residual": gu.dev_u16(inp["residual"]), "routed_in": gu.dev_u16(inp["routed_prev"]),
                "shared_in": gu.dev_u16(inp["shared_prev"]),
                "out_sum": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "routed_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "shared_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "ids": torch.zeros(n, k, dtype=torch.int32, device="cuda")}

    ref = io_new()
    q.moe_decode_layer_batch(d_g, W, ref, n, gmin, q.alloc_batch_workspace(d_g, n))
    torch.cuda.synchronize()
    outs = [[io_new() for _ in range(10)] for _ in range(2)]
    wss = [q.alloc_batch_workspace(d_g, n) for _ in range(2)]
    streams = [torch.cuda.Stream() for _ in range(2)]
    torch.cuda.synchronize()
    errors = []

    def work(i):
        try:
            with torch.cuda.stream(streams[i]):
                for io in outs[i]:
                    q.moe_decode_layer_batch(d_g, W, io, n, gmin, wss[i])
            streams[i].synchronize()
        except Exception as exc:   # reported by the main thread
            errors.append(exc)

    th = [threading.Thread(target=work, args=(i,)) for i in range(2)]
    for t in th:
        t.start()
    for t in th:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in th)
    assert not errors, errors
    torch.cuda.synchronize()
    for i in range(2):
        for c, io in enumerate(outs[i]):
            for key in ("out_sum", "routed_out", "shared_out"):
                assert torch.equal(io[key].view(torch.int16), ref[key].view(torch.int16)), (i, c, key)
            assert torch.equal(io["ids"], ref["ids"]), (i, c)
    print("  20 calls from two threads bit-identical to the single call", flush=True)


def test_tune_group_min_picks_a_candidate(q, orc):
    """The measured group_min choice: one of the candidates, a positive time,
    and outputs afterwards identical to a plain call's with that choice (and
    so with any other: group_min moves work between bit-identical paths)."""
    cfg = wl.CONFIGS["batch"]
    n = 32
    gu.banner(f"group_min tuner: batch {n}, candidates 4 9 16")
    W, _ = _weights(cfg, wl.Q4_K, wl.Q4_K)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_g = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    inp = _inputs(cfg, n)

    def io_new():
        return {"residual": gu.dev_u16(inp["residual"]), "routed_in": gu.dev_u16(inp["routed_prev"]),
                "shared_in": gu.dev_u16(inp["shared_prev"]),
                "out_sum": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "routed_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "shared_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
                "ids": torch.zeros(n, k, dtype=torch.int32, device="cuda")}

    io = io_new()
    ws = q.alloc_batch_workspace(d_g, n)
    torch.cuda.synchronize()
    best, us = q.tune_group_min(d_g, W, io, n, ws, candidates=(4, 9, 16), reps=3)
    torch.cuda.synchronize()
    assert best in (4, 9, 16) and us > 0.0, (best, us)
    for g in (best, 1 if best != 1 else 16):
        ref = io_new()
        q.moe_decode_layer_batch(d_g, W, ref, n, g, q.alloc_batch_workspace(d_g, n))
        torch.cuda.synchronize()
        for key in ("out_sum", "routed_out", "shared_out"):
            assert torch.equal(io[key].view(torch.int16), ref[key].view(torch.int16)), (g, key)
    print(f"  picked group_min {best} at {us:.1f} us per call", flush=True)


def test_tune_group_min_refuses_graph_capture(q, orc):
    """The tuner synchronises its stream, so under graph capture it returns
    MOE_ERR_UNSUPPORTED before enqueueing anything."""
    cfg = SMALL
    gu.banner("group_min tuner under graph capture")
    W, _ = _weights(cfg, wl.Q4_K, wl.Q4_K)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_g = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    n = 4
    inp = _inputs(cfg, n)
    io = {"residual": gu.dev_u16(inp["residual"]), "routed_in": gu.dev_u16(inp["routed_prev"]),
          "shared_in": gu.dev_u16(inp["shared_prev"]),
          "out_sum": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
          "routed_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda"),
          "shared_out": torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")}
    ws = q.alloc_batch_workspace(d_g, n)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with pytest.raises(q.MoeError) as err:
        with torch.cuda.graph(g, stream=s):
            io["out_sum"].zero_()   # one node, so the capture is not empty
            q.tune_group_min(d_g, W, io, n, ws, candidates=(2, 3), reps=1)
    assert err.value.status == -7, err.value
    torch.cuda.synchronize()
    # the device still works: a plain call afterwards
    q.moe_decode_layer_batch(d_g, W, io, n, 2, ws)
    torch.cuda.synchronize()
    assert torch.isfinite(io["routed_out"].float()).all()
