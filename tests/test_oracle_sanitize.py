"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(including float-to-int overflow checks and leak detection): a small C driver runs the stack,
the grouped batch, the top-k on tie-heavy sets, the Q8_1 quantiser and the
load-time requantisation on seeded inputs (Q5_K down and Q8_0 shared, so the
padded down rows and every block type are read), must finish with no
sanitizer report, and must give bit for bit what the normal build gives."""
import os
import shutil
import subprocess

import numpy as np
import pytest
import torch

import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def sanitized(tmp_path_factory):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tmp_path_factory.mktemp("orc_san")
    exe = str(d / "orc_san")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined,float-cast-overflow", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "moe_oracle.c"), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    return exe


def test_oracle_under_sanitizers(orc, sanitized, tmp_path):
    cfg = wl.variant(wl.CONFIGS["tiny"], norm=True, layers=2, config_index=7)
    st, dt = wl.Q8_0, wl.Q5_K
    L, H, E, k, F, Fs = cfg.layers, cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    Ws = [wl.to_numpy_weights(wl.layer_weights(cfg, l, "cpu", shared_type=st, down_type=dt)) for l in range(L)]
    n_tok, n_sets = 3, 200
    rng = np.random.default_rng(5)
    lg = rng.integers(-3, 4, size=(n_sets, E)).astype(np.float32) * np.float32(0.25)
    lg[0] = 0.0
    lg[1, ::2] = -0.0
    q81_x = rng.standard_normal(32 * 8).astype(np.float32)
    q81_x[:32] = 0.0
    q81_x[32:64] = [0.5, 1.5, 2.5, -0.5, -2.5, 127.0] + [0.0] * 26
    inp = wl.u16(wl.token_inputs(cfg, 0)["residual"])
    res = np.stack([wl.u16(wl.randn((H,), wl.seed_for(7, 0, wl.T_INPUT, t)).to(torch.bfloat16)) for t in range(n_tok)])
    rp = np.stack([wl.u16(wl.randn((H,), wl.seed_for(7, 0, wl.T_RPREV, t)).to(torch.bfloat16)) for t in range(n_tok)])
    sp = np.stack([wl.u16(wl.randn((H,), wl.seed_for(7, 0, wl.T_SPREV, t)).to(torch.bfloat16)) for t in range(n_tok)])
    files = {
        "desc.i32": np.array([H, E, k, F, Fs, wl.Q4_K, dt, st, L, n_tok, n_sets], np.int32),
        "norm_w.f32": np.stack([w["norm_w"] for w in Ws]), "router.f32": np.stack([w["router_w"] for w in Ws]),
        "sgw.f32": np.stack([w["shared_gate_w"] for w in Ws]),
        "input.u16": inp, "batch_res.u16": res, "batch_rp.u16": rp, "batch_sp.u16": sp,
        "logits.f32": lg, "q81_x.f32": q81_x,
        "attn.u16": np.stack([wl.u16(wl.attention_output(cfg, 0, l)) for l in range(L)]),
    }
    for name in ("gate", "up", "down", "sgate", "sup", "sdown"):
        files[name + ".u8"] = np.concatenate([w[name].reshape(-1) for w in Ws])
    for n, a in files.items():
        np.ascontiguousarray(a).tofile(str(tmp_path / n))
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sanitized, str(tmp_path)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr[-4000:]

    def got(name, dtype):
        return np.fromfile(str(tmp_path / name), dtype=dtype)

    do = orc.make_desc(H, E, k, F, Fs, down_type=dt, shared_type=st, eps=cfg.eps)
    out, per = orc.moe_stack(do, Ws, inp, per_layer=True)
    assert np.array_equal(got("stack_out.u16", np.uint16), out)
    assert np.array_equal(got("stack_ids.i32", np.int32).reshape(L, k), per["ids"])
    assert np.array_equal(got("stack_attn_out.u16", np.uint16), orc.moe_stack(do, Ws, inp, attn=files["attn.u16"]))
    ob = orc.moe_layer_batch(do, Ws[0], n_tok, residual=res, routed_prev=rp, shared_prev=sp)
    assert np.array_equal(got("batch_routed.u16", np.uint16).reshape(n_tok, H), ob["routed"])
    assert np.array_equal(got("batch_shared.u16", np.uint16).reshape(n_tok, H), ob["shared"])
    tk = got("topk.i32", np.int32).reshape(n_sets, k)
    for s in range(n_sets):
        assert np.array_equal(tk[s], orc.topk(lg[s], k)), s
    assert np.array_equal(got("q81.u8", np.uint8), orc.quantize_q8_1(q81_x))
    Kp = wl.pad_k(dt, F)
    assert np.array_equal(got("requant_down.u8", np.uint8), orc.requant_q4k(Ws[0]["down"], dt, E * H, Kp).reshape(-1))
    assert np.array_equal(got("requant_sgate.u8", np.uint8), orc.requant_q4k(Ws[0]["sgate"], st, Fs, H).reshape(-1))
