"""Parity of the grouped batch path (several tokens, experts grouped) against
the oracle's grouped path.

Stage-isolated: the oracle's own xn, Q8_1 xq, ids, weights and gates go into
expert_ffn_grouped; h of integer-path groups must match the oracle's fp32
values to one rounding (as at batch 1), h of bf16-path groups within the 2e-3
bar (fp32 matrix-core accumulation against an fp64 sum).  The down stage of a
bf16-path group is then checked on identical inputs too: the oracle's bf16
rows applied to the GPU's own h (bf16(h) of two nearly equal h can differ by
a bf16 ulp, so the oracle's h would not be the same input); every bf16 output
must be within the bar of that.  Chained: moe_decode_layer_batch from the raw
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
    return SMALL if name == "small" else wl.CONFIGS[name]


@pytest.mark.parametrize("cfg_name,n,gmin,shared_type,down_type", CASES)
def test_grouped_ffn_stage_isolated(q, orc, cfg_name, n, gmin, shared_type, down_type):
    cfg = _cfg(cfg_name)
    gu.banner(f"grouped ffn {cfg_name} n {n} group_min {gmin} shared {shared_type} down {down_type}")
    W, Wn = _weights(cfg, shared_type, down_type)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_o = orc.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, eps=cfg.eps)
    d_g = q.make_desc(H, E, k, F, Fs, down_type=down_type, shared_type=shared_type, eps=cfg.eps)
    inp = _inputs(cfg, n)
    o = orc.moe_layer_batch(d_o, Wn, n, gmin, **inp)
    ws = q.alloc_batch_workspace(d_g, n)
    routed = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    shared = torch.zeros(n, H, dtype=torch.bfloat16, device="cuda")
    h = torch.zeros(n, k, F, dtype=torch.float32, device="cuda")
    hs = torch.zeros(n, Fs, dtype=torch.float32, device="cuda")
    q.expert_ffn_grouped(d_g, W, gu.dev(o["xn"]), gu.dev(o["xq"]), gu.dev(o["ids"]), gu.dev(o["weights"]),
                         gu.dev(o["shared_gate"]), n, gmin, routed, shared, h, hs, ws)
    torch.cuda.synchronize()
    gh = gu.host(h)
    big = o["group_size"] >= gmin
    if (~big).any():
        gu.assert_f32_within(gh[~big], o["h"][~big], "h (integer path)")
        dh = gu.ulp_diff_f32(gh[~big], o["h"][~big])
        assert (dh > 0).mean() < 1e-3, (dh > 0).sum()
    if big.any():
        gu.assert_f32_within(gh[big], o["h"][big], "h (bf16 path)")
    ghs = gu.host(hs)
    gu.assert_f32_within(ghs, o["hs"], "hs (shared group)")
    # the down stage on identical inputs: bf16-path groups take the GPU's h
    y = o["y"].astype(np.float64).copy()
    Kp = wl.pad_k(down_type, F)
    rb = wl.row_bytes(down_type, Kp)
    down = Wn["down"].reshape(E, H * rb)
    for e in np.unique(o["ids"][big]):
        ts, ss = np.nonzero((o["ids"] == e) & big)
        y[ts, ss] = orc.rows_dot_bf16(down[e], down_type, Kp, H, gh[ts, ss])
    routed_exact = np.einsum("ts,tsh->th", o["weights"].astype(np.float64), y)
    ys = o["ys"].astype(np.float64)
    if n >= gmin:
        Kps = wl.pad_k(shared_type, Fs)
        ys = orc.rows_dot_bf16(Wn["sdown"], shared_type, Kps, H, ghs).astype(np.float64)
    shared_exact = o["shared_gate"].astype(np.float64)[:, None] * ys
    gu.assert_bf16_within(gu.u16_host(routed), routed_exact, "routed")
    gu.assert_bf16_within(gu.u16_host(shared), shared_exact, "shared")
    print(f"  groups >= {gmin}: {int(big.sum())} of {big.size} slots; routed exact "
          f"{float((gu.u16_host(routed) == o['routed']).mean()):.5f}, shared exact "
          f"{float((gu.u16_host(shared) == o['shared']).mean()):.5f}", flush=True)


@pytest.mark.parametrize("cfg_name,n,gmin", [("batch", 8, 4), ("batch", 32, 4), ("small", 12, 3)])
def test_decode_layer_batch_chained(q, orc, cfg_name, n, gmin):
    cfg = _cfg(cfg_name)
    gu.banner(f"decode_layer_batch {cfg_name} n {n} group_min {gmin}")
    W, Wn = _weights(cfg, wl.Q4_K, wl.Q4_K)
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    d_o = orc.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    d_g = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    inp = _inputs(cfg, n)
    o = orc.moe_layer_batch(d_o, Wn, n, gmin, **inp)
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
