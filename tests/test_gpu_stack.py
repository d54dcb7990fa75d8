"""Parity of the persistent L-layer stack (one launch per token)
against the oracle, at the depth the benchmark runs (40 layers of the
Qwen3.6-shaped layer in both weight variants, 48 layers of the 128-expert
shape, with an all-zero token) and on smaller shapes that reach the other code
paths (E > 256 up to 1024, k > 8, few experts, no shared expert, the tiny
shape), with the per-layer stage-isolated and chained checks of
stack_check.py; plus the binding rules, refusals and many launches in a row.
"""
import numpy as np
import pytest
import torch

import gpu_util as gu
import stack_check as sc
import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import quantized_router_expert_amd as q
    assert torch.cuda.is_available()
    return q


def _status(q, desc, L, ws):
    return q.stack_status(desc, L, ws)


FULL_CASES = [
    ("stack", wl.Q4_K, wl.Q4_K, [0, 1, 2], False),
    ("stack", wl.Q8_0, wl.Q5_K, [0, 1, 2], False),
    ("e128", wl.Q4_K, wl.Q4_K, [0, 1, "zero"], False),
    ("stack", wl.Q4_K, wl.Q4_K, [0, 1], True),
    ("stack", wl.Q8_0, wl.Q4_K, [0, 1], False),
    ("stack", wl.Q4_K, wl.Q5_K, [0, 1], False),
    ("e128", wl.Q4_K, wl.Q5_K, [0, "zero"], False),
]


@pytest.mark.parametrize("cfg_name,shared_type,down_type,tokens,attn", FULL_CASES,
                         ids=["stack40-q4k-q4k", "stack40-q8_0-q5k", "e128-48L", "stack40-q4k-q4k-attn",
                              "stack40-q8_0-q4k", "stack40-q4k-q5k", "e128-48L-q5k"])
def test_stack_full_depth_vs_oracle(q, orc, cfg_name, shared_type, down_type, tokens, attn):
    cfg = wl.CONFIGS[cfg_name]
    gu.banner(f"persistent stack {cfg_name} {cfg.layers} layers shared {shared_type} down {down_type} tokens {tokens} "
              f"attention {attn}")
    sc.run_and_check(q, orc, cfg, shared_type, down_type, tokens, q.MOE_STACK_PERSISTENT, with_attn=attn)
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg_name,layers", [("stack", 40), ("e128", 48)])
def test_stack_cooperative_launch_is_the_same(q, cfg_name, layers):
    """MOE_STACK_COOPERATIVE runs the kernel of MOE_STACK_PERSISTENT in a
    cooperative launch: the same bits, token after token, with either launch
    following the other, and status 0."""
    cfg = wl.variant(wl.CONFIGS[cfg_name], layers=layers)
    gu.banner(f"cooperative and plain launches of the {cfg_name} stack, {layers} layers")
    L, H, k = cfg.layers, cfg.H, cfg.k
    Ws = [wl.layer_weights(cfg, l, "cuda") for l in range(L)]
    desc = q.make_desc(H, cfg.E, k, cfg.F, cfg.Fs, eps=cfg.eps)
    ws = q.alloc_workspace(desc, L)
    q.moe_stack_bind(desc, Ws, ws)
    arr = q.layer_array(Ws)
    for t in range(4):
        inp = wl.token_inputs(cfg, t, "cuda")["residual"]
        outs = []
        for mode in ((q.MOE_STACK_PERSISTENT, q.MOE_STACK_COOPERATIVE) if t % 2 == 0
                     else (q.MOE_STACK_COOPERATIVE, q.MOE_STACK_PERSISTENT)):
            out = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
            ids = torch.full((L, k), -1, dtype=torch.int32, device="cuda")
            q.moe_decode_stack(desc, None, inp, out, ids, None, mode, ws, layer_array=arr)
            outs.append((out, ids))
        torch.cuda.synchronize()
        assert _status(q, desc, L, ws) == 0
        assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16)), t
        assert torch.equal(outs[0][1], outs[1][1]), t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kw", [dict(layers=4, E=16), dict(layers=3, E=16, Fs=0, three_input=False)])
def test_stack_behind_attention_small(q, orc, kw):
    """The attention path on the generic instance (every size at run time),
    with and without a shared expert."""
    cfg = wl.variant(wl.CONFIGS["stack"], **kw)
    gu.banner(f"persistent stack behind attention {kw}")
    sc.run_and_check(q, orc, cfg, wl.Q4_K, wl.Q4_K, [0, 1], q.MOE_STACK_PERSISTENT, with_attn=True)


def test_every_benchmark_shape_has_a_compile_time_instance(q):
    """The 40-layer shape in each of its four weight variants and the
    128-expert shape in both of its down variants run compile-time
    instances; a shape outside the table takes the run-time one."""
    gu.banner("persistent instances of the benchmark shapes")
    for st in (wl.Q4_K, wl.Q8_0):
        for dt in (wl.Q4_K, wl.Q5_K):
            assert q.moe_stack_kernel_shape(q.make_desc(2048, 256, 8, 512, 512, down_type=dt, shared_type=st)) == 1
    for dt in (wl.Q4_K, wl.Q5_K):
        assert q.moe_stack_kernel_shape(q.make_desc(2048, 128, 8, 768, 0, down_type=dt)) == 2
    assert q.moe_stack_kernel_shape(q.make_desc(2048, 16, 8, 512, 512)) == 0
    assert q.moe_stack_kernel_shape(q.make_desc(512, 32, 4, 128, 128, norm=0)) == -1


SMALL_CASES = [
    ("stack", dict(layers=4, E=16), wl.Q4_K, wl.Q4_K, [0, 1]),
    ("tiny", dict(layers=3, norm=True), wl.Q4_K, wl.Q4_K, [0, 1, 2]),
    ("tiny", dict(layers=3, norm=True, E=320, router_dup=1), wl.Q4_K, wl.Q4_K, [0, 1]),    # E > 256: per-wave picks
    ("tiny", dict(layers=3, norm=True, k=12), wl.Q4_K, wl.Q4_K, [0, 1]),                   # k > 8: 16 slots per wave
    ("tiny", dict(layers=3, norm=True, E=320, k=16, router_dup=1), wl.Q4_K, wl.Q4_K, [0, 1]),
    ("tiny", dict(layers=3, norm=True, E=1024, k=16, router_dup=1), wl.Q4_K, wl.Q4_K, [0]),
    ("tiny", dict(layers=3, norm=True, Fs=0, three_input=False), wl.Q4_K, wl.Q4_K, [0, 1]),
]


@pytest.mark.parametrize("cfg_name,kw,shared_type,down_type,tokens", SMALL_CASES)
def test_stack_small_shapes_vs_oracle(q, orc, cfg_name, kw, shared_type, down_type, tokens):
    cfg = wl.variant(wl.CONFIGS[cfg_name], **kw)
    gu.banner(f"persistent stack {cfg_name} {kw}")
    Ws, desc, ws, arr = sc.run_and_check(q, orc, cfg, shared_type, down_type, tokens, q.MOE_STACK_PERSISTENT)
    # the per-layer kernel path on the same input chooses the same experts
    L, H, k = cfg.layers, cfg.H, cfg.k
    ws_k = q.alloc_workspace(desc, L)
    inp = wl.token_inputs(cfg, tokens[0], "cuda")["residual"]
    ids_p = torch.full((L, k), -1, dtype=torch.int32, device="cuda")
    ids_k = torch.full_like(ids_p, -1)
    out_p = torch.zeros(H, dtype=torch.bfloat16, device="cuda")
    out_k = torch.zeros_like(out_p)
    q.moe_decode_stack(desc, None, inp, out_p, ids_p, None, q.MOE_STACK_PERSISTENT, ws, layer_array=arr)
    q.moe_decode_stack(desc, None, inp, out_k, ids_k, None, q.MOE_STACK_KERNELS, ws_k, layer_array=arr)
    torch.cuda.synchronize()
    assert torch.equal(ids_p, ids_k)


def test_stack_binding_and_refusals(q, orc):
    """Unbound, bound to other layers, bound correctly; AUTO without a binding
    takes the per-layer kernels; a launch that starts with a nonzero status
    word does no work and leaves the word as it was."""
    cfg = wl.variant(wl.CONFIGS["stack"], layers=2, E=16)
    gu.banner("persistent stack binding and refusals")
    Ws = [wl.layer_weights(cfg, l, "cuda") for l in range(2)]
    desc = q.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs)
    ws = q.alloc_workspace(desc, 2)
    out = torch.zeros(cfg.H, dtype=torch.bfloat16, device="cuda")
    inp = wl.token_inputs(cfg, 0, "cuda")["residual"]
    with pytest.raises(q.MoeError) as e:
        q.moe_decode_stack(desc, Ws, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws)
    assert e.value.status == -8
    # AUTO on the unbound workspace: the per-layer kernels, whose result is the reference
    ref = torch.zeros_like(out)
    ws_k = q.alloc_workspace(desc, 2)
    q.moe_decode_stack(desc, Ws, inp, ref, None, None, q.MOE_STACK_KERNELS, ws_k)
    q.moe_decode_stack(desc, Ws, inp, out, None, None, q.MOE_STACK_AUTO, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, ref) and _status(q, desc, 2, ws) == 0
    # bound to other layers: the caller's table is not the bound one
    Ws2 = [wl.layer_weights(cfg, l + 5, "cuda") for l in range(2)]
    q.moe_stack_bind(desc, Ws2, ws)
    with pytest.raises(q.MoeError) as e:
        q.moe_decode_stack(desc, Ws, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws)
    assert e.value.status == -8
    # a middle layer changed in the caller's table: not the bound stack
    Ws3 = [wl.layer_weights(cfg, l, "cuda") for l in range(3)]
    Ws3b = [Ws3[0], wl.layer_weights(cfg, 7, "cuda"), Ws3[2]]
    ws3 = q.alloc_workspace(desc, 3)
    q.moe_stack_bind(desc, Ws3, ws3)
    with pytest.raises(q.MoeError) as e:
        q.moe_decode_stack(desc, Ws3b, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws3)
    assert e.value.status == -8
    ref3 = torch.zeros_like(out)
    ws3k = q.alloc_workspace(desc, 3)
    q.moe_decode_stack(desc, Ws3b, inp, ref3, None, None, q.MOE_STACK_KERNELS, ws3k)
    q.moe_decode_stack(desc, Ws3b, inp, out, None, None, q.MOE_STACK_AUTO, ws3)
    torch.cuda.synchronize()
    assert torch.equal(out, ref3)
    # the workspace cleared behind the library's back (the host record still
    # names it): the launch finds no bound table on the device and refuses
    ws3.zero_()
    q.moe_decode_stack(desc, Ws3, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws3)
    torch.cuda.synchronize()
    assert _status(q, desc, 3, ws3) == 2 and torch.isnan(out.float()).all()
    # bound correctly: runs, status clear, the same result as the per-layer path's ids
    q.moe_stack_bind(desc, Ws, ws)
    q.moe_decode_stack(desc, Ws, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws)
    torch.cuda.synchronize()
    assert _status(q, desc, 2, ws) == 0 and not torch.isnan(out.float()).any()
    good = out.clone()
    # a nonzero status word set from the host: refused, output NaN, word unchanged
    off = q.moe_stack_status_offset(desc, 2)
    ws[off:off + 4].view(torch.int32).fill_(1)
    q.moe_decode_stack(desc, Ws, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws)
    torch.cuda.synchronize()
    assert _status(q, desc, 2, ws) == 1 and torch.isnan(out.float()).all()
    q.moe_decode_stack(desc, Ws, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws)
    torch.cuda.synchronize()
    assert _status(q, desc, 2, ws) == 1 and torch.isnan(out.float()).all()
    # re-binding clears it
    q.moe_stack_bind(desc, Ws, ws)
    q.moe_decode_stack(desc, Ws, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws)
    torch.cuda.synchronize()
    assert _status(q, desc, 2, ws) == 0 and torch.equal(out, good)
    # moe_workspace_init drops the host record
    q.moe_workspace_init(ws)
    with pytest.raises(q.MoeError) as e:
        q.moe_decode_stack(desc, Ws, inp, out, None, None, q.MOE_STACK_PERSISTENT, ws)
    assert e.value.status == -8


def test_stack_many_tokens_deterministic(q):
    """200 launches in a row on one workspace (the generation counter advances
    each launch): the same input gives the same output every time, and the
    status word stays 0."""
    cfg = wl.variant(wl.CONFIGS["stack"], layers=4)
    gu.banner("persistent stack: 200 launches")
    Ws = [wl.layer_weights(cfg, l, "cuda") for l in range(4)]
    desc = q.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs)
    ws = q.alloc_workspace(desc, 4)
    q.moe_stack_bind(desc, Ws, ws)
    arr = q.layer_array(Ws)
    inps = [wl.token_inputs(cfg, t, "cuda")["residual"] for t in range(3)]
    outs = torch.zeros(200, cfg.H, dtype=torch.bfloat16, device="cuda")
    for i in range(200):
        q.moe_decode_stack(desc, None, inps[i % 3], outs[i], None, None, q.MOE_STACK_PERSISTENT, ws, layer_array=arr)
    torch.cuda.synchronize()
    assert _status(q, desc, 4, ws) == 0
    for i in range(3, 200):
        assert torch.equal(outs[i], outs[i % 3]), i
