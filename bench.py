"""Benchmark: batch-1 decode MoE stage of a Qwen3.6-35B-A3B-shaped model on one MI355X.

One step = one decode token through the 40-layer MoE stack (residual-add +
RMSNorm, fp32 router over 256 experts, top-8 + softmax, Q4_K x Q8_1 routed
gate/up + SwiGLU + down, sigmoid-gated shared expert), tokens strictly in
sequence on one stream.  Weights (18 GB of Q4_K routed experts + router +
shared) and the 128 token inputs are generated from seeds and resident in HBM
before timing.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 128] [--warmup 8] [--mode auto|kernels|persistent]
                  [--variant after|before|both] [--no-cpu] [--no-batch] [--no-requant]
                  [--no-e128] [--no-layer] [--no-attn] [--calib-copy] [--trace]
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=128)
    p.add_argument("--warmup", type=int, default=8)
    p.add_argument("--mode", default="auto", choices=["auto", "kernels", "persistent"])
    p.add_argument("--variant", default="both", choices=["after", "before", "both"])
    p.add_argument("--layers", type=int, default=40)
    p.add_argument("--tokens", type=int, default=128)
    p.add_argument("--repeats", type=int, default=5)
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--no-batch", action="store_true", help="skip the grouped batch-path leg")
    p.add_argument("--no-requant", action="store_true", help="skip the load-time requantisation leg")
    p.add_argument("--no-e128", action="store_true", help="skip the 128-expert 48-layer stack leg")
    p.add_argument("--no-layer", action="store_true", help="skip the single-layer moe_decode_layer leg")
    p.add_argument("--no-attn", action="store_true", help="skip the stack-behind-attention leg")
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--cpu-seconds-1t", type=float, default=6.0, help="single-thread oracle time")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a kernel that reads and writes 1 GiB each (HBM counter calibration)")
    p.add_argument("--trace", action="store_true", help="print the persistent kernel's per-phase times to stderr")
    return p.parse_args()


def algorithmic_bytes(cfg, shared_type, down_type):
    """Bytes the method must read per token: router, norm weight, shared-gate row
    (with a shared expert), the k selected experts' gate/up/down rows and the
    shared expert, per layer."""
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    per = 4 * E * H + 4 * H + (4 * H if Fs else 0)   # router, norm weight, shared-gate row
    per += k * 2 * F * wl.row_bytes(wl.Q4_K, H)
    per += k * H * wl.row_bytes(down_type, wl.pad_k(down_type, F))
    if Fs:
        per += 2 * Fs * wl.row_bytes(shared_type, H) + H * wl.row_bytes(shared_type, wl.pad_k(shared_type, Fs))
    return per * cfg.layers


class Stack:
    """40 layers of weights on the GPU plus everything one token needs
    (with_attn: a seeded attention-block output per token and layer, which
    each layer adds to the folded residual before its norm)."""

    def __init__(self, q, cfg, shared_type, down_type, mode, with_attn=False):
        self.q, self.cfg = q, cfg
        self.shared_type, self.down_type = shared_type, down_type
        t0 = time.time()
        self.layers = [wl.layer_weights(cfg, l, "cuda", shared_type=shared_type, down_type=down_type)
                       for l in range(cfg.layers)]
        torch.cuda.synchronize()
        self.gen_s = time.time() - t0
        self.desc = q.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs, down_type=down_type, shared_type=shared_type,
                                eps=cfg.eps)
        self.arr = q.layer_array(self.layers)
        self.ws = q.alloc_workspace(self.desc, cfg.layers)
        self.inputs = torch.stack([wl.token_inputs(cfg, t, "cuda")["residual"] for t in range(cfg.tokens)])
        self.attn = None
        if with_attn:
            self.attn = torch.stack([torch.stack([wl.attention_output(cfg, t, l, "cuda") for l in range(cfg.layers)])
                                     for t in range(cfg.tokens)]).contiguous()
        self.out = torch.zeros(cfg.tokens, cfg.H, dtype=torch.bfloat16, device="cuda")
        self.ids = torch.zeros(cfg.layers, cfg.k, dtype=torch.int32, device="cuda")
        self.mode = self._pick_mode(mode)
        self.graphs = None
        if self.mode == q.MOE_STACK_KERNELS:
            self._capture()

    def _pick_mode(self, mode):
        q = self.q
        if mode in ("auto", "persistent"):
            try:
                q.moe_stack_bind(self.desc, self.layers, self.ws)
                self.run_eager(0, q.MOE_STACK_PERSISTENT)
                torch.cuda.synchronize()
                return q.MOE_STACK_PERSISTENT
            except q.MoeError as e:
                if mode == "persistent":
                    raise
                print(f"# persistent mode unavailable ({e}); using per-layer kernels in HIP graphs", file=sys.stderr)
        return q.MOE_STACK_KERNELS

    def run_eager(self, t, mode, ids=None):
        self.q.moe_decode_stack(self.desc, None, self.inputs[t], self.out[t], ids, None, mode, self.ws,
                                layer_array=self.arr, attn=None if self.attn is None else self.attn[t])

    def _capture(self):
        """One HIP graph per token input (4 kernels per layer + the final fold)."""
        s = torch.cuda.Stream()
        self.stream = s
        torch.cuda.synchronize()   # the inputs are made on the default stream
        with torch.cuda.stream(s):
            self.run_eager(0, self.q.MOE_STACK_KERNELS)
        s.synchronize()
        self.graphs = []
        for t in range(self.cfg.tokens):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                self.run_eager(t, self.q.MOE_STACK_KERNELS)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def step(self, t):
        t %= self.cfg.tokens
        if self.graphs is not None:
            self.graphs[t].replay()
        else:
            self.run_eager(t, self.mode)


def time_steps(stack, steps, warmup, repeats):
    for i in range(warmup):
        stack.step(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    per_token_us = []
    for r in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(steps):
            stack.step(i)
        e1.record(stream)
        torch.cuda.synchronize()
        per_token_us.append(e0.elapsed_time(e1) * 1e3 / steps)
    return per_token_us


def layer_leg(q, layers=None, n_inputs=128, repeats=5):
    """Qwen3.6-shaped layers (H 2048, 256 experts top-8, F 512, shared 512,
    Q4_K) through the per-layer entry point moe_decode_layer, batch 1, on
    n_inputs fresh seeded inputs (residual, previous routed and shared
    outputs ~N(0,1) bf16), input i on layer i mod len(layers) (the stack's
    layers when given, else one layer of its own), each input's call
    captured in its own HIP graph and the graphs replayed back to back:
    microseconds per layer call (median of `repeats` passes), and GB/s over
    the bytes the layer must read (router, norm weight, shared-gate row, the
    8 selected experts, the shared expert).  With the 40 layers of the stack,
    a layer's router and shared expert come back after 39 other layers'
    calls, as in a decode step; with one layer they stay in the last-level
    cache between calls."""
    cfg = wl.CONFIGS["layer"]
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    W = None
    if not layers:
        W = wl.layer_weights(cfg, 0, "cuda")
        layers = [W]
    desc = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    lws = [q.make_weights(L) for L in layers]
    nl = len(lws)
    ws = q.alloc_workspace(desc)
    ios = []
    for t in range(n_inputs):
        ti, pv = wl.token_inputs(cfg, t, "cuda"), wl.prev_outputs(cfg, t, "cuda")
        ios.append({"residual": ti["residual"], "routed_in": pv["routed_prev"], "shared_in": pv["shared_prev"],
                    "out_sum": torch.empty(H, dtype=torch.bfloat16, device="cuda"),
                    "routed_out": torch.empty(H, dtype=torch.bfloat16, device="cuda"),
                    "shared_out": torch.empty(H, dtype=torch.bfloat16, device="cuda")})
    s = torch.cuda.Stream()
    torch.cuda.synchronize()   # the inputs are made on the default stream
    with torch.cuda.stream(s):
        q.moe_decode_layer(desc, lws[0], ios[0], ws)
    s.synchronize()
    graphs = []
    for i, io in enumerate(ios):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            q.moe_decode_layer(desc, lws[i % nl], io, ws)
        graphs.append(g)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    for g in graphs[:8]:
        g.replay()
    us = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for g in graphs:
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us.append(e0.elapsed_time(e1) * 1e3 / n_inputs)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i, io in enumerate(ios):
        q.moe_decode_layer(desc, lws[i % nl], io, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    eager = e0.elapsed_time(e1) * 1e3 / n_inputs
    # all the calls in one graph, the way a decode step captures its layers
    g_all = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_all, stream=s):
        for i, io in enumerate(ios):
            q.moe_decode_layer(desc, lws[i % nl], io, ws)
    torch.cuda.synchronize()
    g_all.replay()
    us_one = []
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        g_all.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us_one.append(e0.elapsed_time(e1) * 1e3 / n_inputs)
    one = float(np.median(us_one))
    med = float(np.median(us))
    nbytes = algorithmic_bytes(cfg, wl.Q4_K, wl.Q4_K)
    res = {"workload": f"Qwen3.6-shaped layers through moe_decode_layer, batch 1, {n_inputs} fresh inputs, input i "
                       f"on layer i mod {nl}, one HIP graph per input replayed back to back", "layers_rotated": nl,
           "us_per_layer": med, "us_p10": float(np.percentile(us, 10)), "us_p90": float(np.percentile(us, 90)),
           "us_per_layer_eager": eager, "us_per_layer_one_graph": one,
           "alg_bytes_per_layer": nbytes, "achieved_GBs": nbytes / (med * 1e-6) / 1e9}
    res["frac_of_peak"] = res["achieved_GBs"] / HBM_PEAK_GBS
    print(f"# layer (moe_decode_layer in graphs, {nl} layers rotated): {med:.1f} us per layer "
          f"({res['achieved_GBs']:.0f} GB/s); "
          f"eager {eager:.1f} us; all {n_inputs} calls in one graph {one:.1f} us", file=sys.stderr, flush=True)
    del graphs, g_all, W
    torch.cuda.empty_cache()
    return res


def check_against_kernels(q, stack, t=0):
    """The timed path's output for token t against the per-layer kernel path
    on the same input (another summation order, so rare last-bit
    differences): fraction of equal bf16 outputs and relative L2 distance."""
    if stack.mode != q.MOE_STACK_PERSISTENT:
        return None
    ws_k = q.alloc_workspace(stack.desc, stack.cfg.layers)
    out_p = torch.zeros(stack.cfg.H, dtype=torch.bfloat16, device="cuda")
    out_k = torch.zeros_like(out_p)
    stack.q.moe_decode_stack(stack.desc, None, stack.inputs[t], out_p, None, None, q.MOE_STACK_PERSISTENT, stack.ws,
                             layer_array=stack.arr)
    stack.q.moe_decode_stack(stack.desc, None, stack.inputs[t], out_k, None, None, q.MOE_STACK_KERNELS, ws_k,
                             layer_array=stack.arr)
    torch.cuda.synchronize()
    a, b = out_p.double(), out_k.double()
    rel = float((a - b).norm() / b.norm())
    del ws_k
    return {"token": t, "bits_equal_frac": float((out_p.view(torch.int16) == out_k.view(torch.int16)).float().mean()),
            "rel_l2": rel}


def require_status_ok(q, stack, what):
    """The persistent kernel's status word must be 0 after the timed launches
    (1: a launch stopped at a bounded wait; 2: the bound table was not the
    caller's; 3: a die number outside 0..7); otherwise
    the run is invalid and the benchmark stops."""
    if stack.mode != q.MOE_STACK_PERSISTENT:
        return
    st = q.stack_status(stack.desc, stack.cfg.layers, stack.ws)
    if st != 0:
        detail = q.stack_stop_detail(stack.desc, stack.cfg.layers, stack.ws) if st == 1 else None
        print(json.dumps({"error": f"{what}: persistent stack status word {st} after the timed launches",
                          "stop_layer_check": detail}))
        sys.exit(1)


def batch_leg(q, sizes=(8, 32), group_min=9, n_layers=6, rounds=5, tune=(6, 9, 12)):
    """The grouped batch path on layers of the 40-layer shape: per batch size,
    microseconds per layer step (norm, router, grouped experts, combine), with
    `n_layers` layers, each with its own weights and its own seeded batch
    (inputs ~N(0,1), a quarter of the tokens steered to two experts of that
    layer), one HIP graph per layer step, replayed in layer order `rounds`
    times.  A layer's weights come back only after the other layers' steps
    (at least 5 x 108 MB at batch 8), more than the 256 MB last-level cache
    holds, as in a decode step where each layer's weights are read once.
    Reports tokens/s and GB/s over the bytes a step must read (router, shared
    expert, each distinct selected expert once; averaged over the layers).
    group_min: groups of that many tokens or more take the int8 matrix cores,
    whose tile is 16 tokens.  With `tune`, moe_tune_group_min picks it among
    those candidates on this device (9 has been the measured best at batch 8
    and 32 among 4, 6, 9, 12 and 16); group_min changes no output bit."""
    cfg = wl.CONFIGS["batch"]
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    desc = q.make_desc(H, E, k, F, Fs, eps=cfg.eps)
    Ws = [wl.layer_weights(cfg, l, "cuda") for l in range(n_layers)]
    lws = [q.make_weights(W) for W in Ws]
    per_expert = 2 * F * wl.row_bytes(wl.Q4_K, H) + H * wl.row_bytes(wl.Q4_K, wl.pad_k(wl.Q4_K, F))
    fixed = 4 * E * H + 4 * H + 4 * H + 2 * Fs * wl.row_bytes(wl.Q4_K, H) + H * wl.row_bytes(wl.Q4_K, Fs)
    out = {}
    s = torch.cuda.Stream()
    for n in sizes:
        ws = q.alloc_batch_workspace(desc, n)
        ios = []
        for l in range(n_layers):
            inp, _, _ = wl.batch_inputs(cfg, n, "cuda", layer=l)
            ios.append({"residual": inp["residual"].contiguous(), "routed_in": inp["routed_prev"].contiguous(),
                        "shared_in": inp["shared_prev"].contiguous(),
                        "out_sum": torch.empty(n, H, dtype=torch.bfloat16, device="cuda"),
                        "routed_out": torch.empty(n, H, dtype=torch.bfloat16, device="cuda"),
                        "shared_out": torch.empty(n, H, dtype=torch.bfloat16, device="cuda"),
                        "ids": torch.empty(n, k, dtype=torch.int32, device="cuda")})
        torch.cuda.synchronize()   # the inputs are made on the default stream
        gmin = group_min
        if tune:   # measured choice on this device (outputs do not depend on it)
            with torch.cuda.stream(s):
                gmin, _ = q.tune_group_min(desc, lws[0], ios[0], n, ws, candidates=tune, reps=5)
            s.synchronize()
        with torch.cuda.stream(s):
            for l in range(n_layers):
                q.moe_decode_layer_batch(desc, lws[l], ios[l], n, gmin, ws)
        s.synchronize()
        graphs = []
        for l in range(n_layers):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                q.moe_decode_layer_batch(desc, lws[l], ios[l], n, gmin, ws)
            graphs.append(g)
        torch.cuda.synchronize()
        for g in graphs:
            g.replay()
        stream = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(rounds):
            for g in graphs:
                g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / (rounds * n_layers)
        distinct = [len(set(io["ids"].flatten().tolist())) for io in ios]   # as the replays selected
        nbytes = fixed + float(np.mean(distinct)) * per_expert
        out[f"batch{n}"] = {"us_per_layer_step": us, "tokens_per_s_per_layer": n * 1e6 / us,
                            "distinct_experts_mean": float(np.mean(distinct)), "distinct_experts": distinct,
                            "bytes_per_step": nbytes, "achieved_GBs": nbytes / (us * 1e-6) / 1e9,
                            "group_min": gmin, "group_min_candidates": list(tune) if tune else None,
                            "layers_rotated": n_layers}
        print(f"# batch {n}: {us:.1f} us per layer step over {n_layers} layers, {np.mean(distinct):.1f} distinct "
              f"experts per layer, {out[f'batch{n}']['achieved_GBs']:.0f} GB/s (group_min {gmin})", file=sys.stderr,
              flush=True)
        del graphs, ws
    del Ws, lws
    torch.cuda.empty_cache()
    return out


def attn_leg(q, steps, warmup, repeats):
    """The 40-layer stack (Q4_K shared and down) behind an attention block per
    layer: each layer adds a seeded bf16 attention output to the folded
    residual (the post-attention add-norm) before its norm.  Timed like the
    primary stack."""
    cfg = wl.CONFIGS["stack"]
    stack = Stack(q, cfg, wl.Q4_K, wl.Q4_K, "auto", with_attn=True)
    us = time_steps(stack, steps, warmup, repeats)
    med = float(np.median(us))
    alg = algorithmic_bytes(cfg, wl.Q4_K, wl.Q4_K)
    require_status_ok(q, stack, "attn")
    res = {"workload": f"{cfg.layers}-layer stack as the primary one, each layer behind an attention block's seeded "
                       "bf16 output (post-attention add-norm before the MoE norm)",
           "us_per_token": med, "us_p10": float(np.percentile(us, 10)), "us_p90": float(np.percentile(us, 90)),
           "tokens_per_s": 1e6 / med, "achieved_GBs": alg / (med * 1e-6) / 1e9,
           "mode": "persistent" if stack.mode == q.MOE_STACK_PERSISTENT else "kernels"}
    print(f"# attn: {med:.1f} us/token", file=sys.stderr, flush=True)
    del stack
    torch.cuda.empty_cache()
    return res


def e128_leg(q, steps, warmup, repeats):
    """The 128-expert variant with no shared expert: 48 layers, H 2048, top-8,
    F 768 (Q4_K gate/up/down), 2-input fold, router rows duplicated in groups of
    4, a tenth of the 128 tokens all zero.  Timed like the primary stack."""
    cfg3 = wl.CONFIGS["e128"]
    stack = Stack(q, cfg3, wl.Q4_K, wl.Q4_K, "auto")
    us = time_steps(stack, steps, warmup, repeats)
    med = float(np.median(us))
    alg = algorithmic_bytes(cfg3, wl.Q4_K, wl.Q4_K)
    launch = launch_durations(stack, min(64, steps))
    require_status_ok(q, stack, "e128")
    check = check_against_kernels(q, stack)
    res = {"workload": f"128-expert variant: {cfg3.layers} layers, H 2048, 128 experts top-8, F 768, no shared "
                       f"expert, batch 1, {cfg3.tokens} sequential tokens",
           "us_per_token": med, "us_p10": float(np.percentile(us, 10)), "us_p90": float(np.percentile(us, 90)),
           "tokens_per_s": 1e6 / med, "alg_bytes_per_token": alg, "achieved_GBs": alg / (med * 1e-6) / 1e9,
           "us_per_layer": med / cfg3.layers, "launch_us": launch, "kernel_GBs": alg / (launch * 1e-6) / 1e9,
           "mode": "persistent" if stack.mode == q.MOE_STACK_PERSISTENT else "kernels", "output_check": check}
    res["frac_of_peak"] = res["kernel_GBs"] / HBM_PEAK_GBS
    res["traffic_bytes_per_launch"] = (measured_traffic("moe_stack_48L_e128_traffic")
                                       if res["mode"] == "persistent" else None)
    print(f"# e128: generated {cfg3.layers} layers in {stack.gen_s:.1f}s; {med:.1f} us/token "
          f"({res['achieved_GBs']:.0f} GB/s)", file=sys.stderr, flush=True)
    del stack
    torch.cuda.empty_cache()
    return res


def launch_durations(stack, n):
    """Average duration of one launch of the step's kernel (one token), from
    events recorded around each launch on the stream the kernel runs on."""
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        ev[i][0].record(stream)
        stack.step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) * 1e3 for a, b in ev]))


KERNEL_SOURCES = ["quantized_router_expert_amd/csrc/moe_stack.hip", "quantized_router_expert_amd/csrc/moe_stack.h",
                  "quantized_router_expert_amd/csrc/moe_device.h", "quantized_router_expert_amd/csrc/moe_select.h"]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(summary):
    """HBM bytes per launch of the persistent kernel from the committed counter
    summary profiles/<summary>.md (FETCH_SIZE + WRITE_SIZE, scaled by a
    copy-kernel calibration), or None when that summary was taken on other
    kernel sources."""
    path = os.path.join(ROOT, "profiles", f"{summary}.md")
    try:
        text = open(path).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if ":" in line and line.strip().startswith("- "):
            k, v = line.strip()[2:].split(":", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel source sha256") != kernel_source_hash():
        return None
    try:
        return float(vals["HBM bytes per launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(stack, seconds, seconds_1t):
    """The oracle, as it stands, on the host cores: whole tokens through the
    40-layer stack, same weights and inputs, until `seconds` have passed; then
    the same on one thread for `seconds_1t`."""
    import oracle as orc
    cfg = stack.cfg
    t0 = time.time()
    Wn = [wl.to_numpy_weights(w) for w in stack.layers]
    copy_s = time.time() - t0
    d = orc.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs, down_type=stack.down_type,
                      shared_type=stack.shared_type, eps=cfg.eps)
    inputs = [wl.u16(stack.inputs[t]) for t in range(cfg.tokens)]

    outs = {}

    def run(limit):
        n = 0
        t0 = time.time()
        while True:
            outs[n % cfg.tokens] = orc.moe_stack(d, Wn, inputs[n % cfg.tokens])
            n += 1
            if time.time() - t0 >= limit or n >= cfg.tokens:
                break
        return (time.time() - t0) / n * 1e6, n

    threads = orc.num_threads()
    us, n = run(seconds)
    orc.set_threads(1)
    us1, n1 = run(seconds_1t)
    orc.set_threads(threads)
    # the timed path's outputs for the same tokens, computed again here (a short
    # timed run need not have reached every token)
    gout = torch.zeros(cfg.tokens, cfg.H, dtype=torch.bfloat16, device="cuda")
    for t in outs:
        stack.q.moe_decode_stack(stack.desc, None, stack.inputs[t], gout[t], None, None, stack.mode, stack.ws,
                                 layer_array=stack.arr)
    torch.cuda.synchronize()
    g = gout.view(torch.int16).cpu().numpy().view(np.uint16)
    eq, rels = [], []
    for t, o in outs.items():
        a = (g[t].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        b = (o.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        eq.append(float((g[t] == o).mean()))
        rels.append(float(np.linalg.norm(a - b) / np.linalg.norm(b)))
    check = {"tokens": len(outs), "bits_equal_frac_min": min(eq), "bits_equal_frac_mean": float(np.mean(eq)),
             "rel_l2_max": max(rels)}
    return {"us_per_token": us, "tokens": n, "threads": threads, "copy_s": copy_s,
            "us_per_token_1t": us1, "tokens_1t": n1, "output_check": check}


def stream_read_gbs(q, n_bytes=4 << 30, reps=10, blocks=512):
    """Achievable HBM read bandwidth from a plain read kernel (the library's
    moe_stream_read: every 16-byte word of a 4 GiB buffer read once)."""
    x = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    out = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    q.moe_stream_read(x, n_bytes, out, blocks)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        q.moe_stream_read(x, n_bytes, out, blocks)
    e1.record()
    torch.cuda.synchronize()
    s = e0.elapsed_time(e1) / 1e3 / reps
    del x, out
    torch.cuda.empty_cache()
    return n_bytes / s / 1e9


def cold_tokens(stack, n, evict_bytes=1 << 30):
    """Per-token latency with the caches flushed: a 1 GiB buffer is streamed
    (read and written) before every token, outside the per-token events."""
    buf = torch.ones(evict_bytes // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for t in range(n):
        buf.mul_(1.0)
        ev[t][0].record(stream)
        stack.step(t % stack.cfg.tokens)
        ev[t][1].record(stream)
    torch.cuda.synchronize()
    us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    del buf
    torch.cuda.empty_cache()
    return float(np.median(us))


def requant_leg(q, reps=20):
    """Load-time requantisation to Q4_K of one layer of the 40-layer shape:
    the 256 routed down matrices from Q5_K and the shared expert's three
    matrices from Q8_0.  Reports time and HBM rate (source read + Q4_K
    written) per call, and the time for all 40 layers."""
    cfg = wl.CONFIGS["stack"]
    W = wl.layer_weights(cfg, 0, "cuda", shared_type=wl.Q8_0, down_type=wl.Q5_K)
    jobs = [("down", wl.Q5_K, cfg.E * cfg.H, cfg.F), ("sgate", wl.Q8_0, cfg.Fs, cfg.H),
            ("sup", wl.Q8_0, cfg.Fs, cfg.H), ("sdown", wl.Q8_0, cfg.H, cfg.Fs)]
    out = {}
    total_us = 0.0
    for name, st, rows, K in jobs:
        src = W[name]
        dst = torch.empty(rows * (K // 256) * 144, dtype=torch.uint8, device="cuda")
        q.moe_requant_q4k(src, st, rows, K, dst)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            q.moe_requant_q4k(src, st, rows, K, dst)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        nbytes = src.numel() + dst.numel()
        out[name] = {"src_type": st, "rows": rows, "K": K, "us": us, "GBs": nbytes / (us * 1e-6) / 1e9,
                     "src_bytes": src.numel(), "dst_bytes": dst.numel()}
        total_us += us
        del dst
    del W
    torch.cuda.empty_cache()
    out["layer_us"] = total_us
    out["model_40_layers_ms"] = total_us * cfg.layers / 1e3
    print(f"# requant to Q4_K, one layer: {total_us:.0f} us (routed down {out['down']['GBs']:.0f} GB/s); "
          f"40 layers {out['model_40_layers_ms']:.1f} ms", file=sys.stderr, flush=True)
    return out


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": f"--gpus {a.gpus}: this benchmark runs on one GPU only; the stage is a batch-1 "
                                   "decode step whose multi-GPU sharding is not built"}))
        sys.exit(2)
    if a.calib_copy:
        # a plain streaming kernel of known traffic for scaling the HBM byte
        # counters: reads 1 GiB and writes 1 GiB (an elementwise kernel, not a
        # copy-engine transfer, so the counters see it)
        n = 1 << 28
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"calib_read_bytes": 4 * n, "calib_write_bytes": 4 * n, "launches": 5}))
        return
    import quantized_router_expert_amd as q
    torch.cuda.set_device(0)
    cfg = wl.variant(wl.CONFIGS["stack"], layers=a.layers, tokens=a.tokens)
    variants = {"after": (wl.Q4_K, wl.Q4_K), "before": (wl.Q8_0, wl.Q5_K)}
    order = ["after", "before"] if a.variant == "both" else [a.variant]
    results = {}
    primary = None
    for name in order:
        st, dt = variants[name]
        stack = Stack(q, cfg, st, dt, a.mode)
        print(f"# {name}: generated {cfg.layers} layers in {stack.gen_s:.1f}s; mode "
              f"{'persistent' if stack.mode == q.MOE_STACK_PERSISTENT else 'kernels+graphs'}", file=sys.stderr, flush=True)
        us = time_steps(stack, a.steps, a.warmup, a.repeats)
        med = float(np.median(us))
        alg = algorithmic_bytes(cfg, st, dt)
        res = {"us_per_token": med, "us_p10": float(np.percentile(us, 10)), "us_p90": float(np.percentile(us, 90)),
               "tokens_per_s": 1e6 / med, "alg_bytes_per_token": alg, "achieved_GBs": alg / (med * 1e-6) / 1e9,
               "us_per_layer": med / cfg.layers, "mode": "persistent" if stack.mode == q.MOE_STACK_PERSISTENT else "kernels"}
        res["frac_of_peak"] = res["achieved_GBs"] / HBM_PEAK_GBS
        res["launch_us"] = launch_durations(stack, min(64, a.steps))
        require_status_ok(q, stack, name)
        res["output_check"] = check_against_kernels(q, stack)
        res["kernel_GBs"] = alg / (res["launch_us"] * 1e-6) / 1e9
        res["traffic_bytes_per_launch"] = (measured_traffic(f"moe_stack_40L_{name}_traffic")
                                           if res["mode"] == "persistent" else None)
        res["cold_us_per_token"] = cold_tokens(stack, 32)
        if a.trace and stack.mode == q.MOE_STACK_PERSISTENT:
            # one more token with every workgroup stamping its events (the timed
            # launches above ran without the per-workgroup stamps)
            for t in range(3):
                q.moe_decode_stack(stack.desc, None, stack.inputs[t], stack.out[t], None, None,
                                   q.MOE_STACK_PERSISTENT, stack.ws, layer_array=stack.arr, trace=1)
            torch.cuda.synchronize()
            tr, mhz = q.stack_trace(stack.desc, cfg.layers, stack.ws)
            tr = tr[1:]   # layer 0 has no previous outputs to wait for
            d = (tr[:, 1:10] - tr[:, :9]).mean(0).tolist()
            names = ["prev outputs in", "fixed weights landed", "norm+router+shared gate/up", "experts selected",
                     "routed gate/up landed", "gate/up compute", "h quantised (exchange)", "down rows landed",
                     "down+combine"]
            print(f"# {name} per-layer phases (us, mean over layers 1..): " +
                  ", ".join(f"{n} {v:.2f}" for n, v in zip(names, d)) + f"; layer {tr[:, 9].mean():.2f}"
                  + f"; shader clock {mhz:.0f} MHz", file=sys.stderr, flush=True)
            bt = q.stack_block_trace(stack.desc, cfg.layers, stack.ws)
            # layer l's events against the moment the last workgroup stored layer l-1's outputs
            ref = bt[:-1, :, 10].max(1).values
            order = [0, 1, 2, 11, 12, 3, 4, 13, 5, 6, 15, 7, 14, 8, 9, 10]
            rel = bt[1:, :, order] - ref[:, None, None]
            ev = ["start", "t in", "fixed", "normed", "xq", "logits out", "hs out", "lg in", "sel", "gu landed",
                  "dn queued", "h out", "h in", "hq", "dn landed", "t out"]
            print("#   all workgroups, from the last t of the previous layer: " +
                  ", ".join(f"{n} {m:.2f}/{x:.2f}" for n, m, x in
                            zip(ev, rel.median(1).values.mean(0).tolist(), rel.max(1).values.mean(0).tolist())) +
                  "  (median/max over workgroups)", file=sys.stderr, flush=True)
        if name == "after":
            primary = (stack, res)
        else:
            del stack
            torch.cuda.empty_cache()
        results[name] = res
        print(f"# {name}: {med:.1f} us/token ({res['achieved_GBs']:.0f} GB/s)", file=sys.stderr, flush=True)
    stack, res = primary if primary else (None, results[order[0]])
    same_shape = primary is not None and cfg.H == wl.CONFIGS["layer"].H and cfg.E == wl.CONFIGS["layer"].E
    layer = None if a.no_layer else layer_leg(q, primary[0].layers if same_shape else None)
    attn = None if a.no_attn else attn_leg(q, a.steps, a.warmup, a.repeats)
    e128 = None if a.no_e128 else e128_leg(q, a.steps, a.warmup, a.repeats)
    batch = None if a.no_batch else batch_leg(q)
    requant = None if a.no_requant else requant_leg(q)
    cpu = None
    if not a.no_cpu and stack is not None:
        c = cpu_baseline(stack, a.cpu_seconds, a.cpu_seconds_1t)
        cpu = {"value": c["us_per_token"], "unit": "us/token", "cores": c["threads"], "kind": "oracle",
               "sample": f"{c['tokens']} whole tokens through the {cfg.layers}-layer stack (same weights and inputs)",
               "single_thread": {"value": c["us_per_token_1t"], "unit": "us/token", "cores": 1,
                                 "sample": f"{c['tokens_1t']} whole tokens"},
               "cpu_model": cpu_model(),
               "achieved_GBs": res["alg_bytes_per_token"] / (c["us_per_token"] * 1e-6) / 1e9,
               "gpu_output_vs_oracle": c["output_check"]}
        if c["output_check"]["rel_l2_max"] > 2e-3:
            print(json.dumps({"error": "timed outputs differ from the oracle's", "check": c["output_check"]}))
            sys.exit(1)
    kernel = "moe_stack_persistent" if res["mode"] == "persistent" else "per-token graph of per-layer kernels"
    line = {
        "metric": "MoE decode stage latency (us/token, 40 layers) + achieved HBM GB/s vs peak",
        "value": res["us_per_token"], "unit": "us/token", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": res["us_per_token"] / 1e3, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "q4_k x q8_1 (int8 dot), fp64 accumulate, bf16 out", "data": "synthetic",
        "config": {"workload": f"Qwen3.6-35B-A3B-shaped MoE stack: {cfg.layers} layers, H 2048, 256 experts top-8, "
                               f"F 512, shared 512, batch 1; timed: {a.steps} sequential tokens per pass (inputs "
                               f"cycling through {cfg.tokens} seeded N(0,1) tokens), {a.repeats} passes, median",
                   "variant": "shared Q4_K + routed down Q4_K", "parallelism": "none (1 GPU)"},
        "tokens_per_s": res["tokens_per_s"], "achieved_GBs": res["achieved_GBs"],
        "us_per_layer": res["us_per_layer"], "us_p10": res["us_p10"], "us_p90": res["us_p90"],
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": res["kernel_GBs"], "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": res["kernel_GBs"] / HBM_PEAK_GBS,
                     "traffic": res["traffic_bytes_per_launch"],
                     # measured HBM bytes (committed counter summary) over the same launch time
                     "traffic_GBs": (res["traffic_bytes_per_launch"] / (res["launch_us"] * 1e-6) / 1e9
                                     if res["traffic_bytes_per_launch"] else None),
                     "alg_bytes_per_launch": res["alg_bytes_per_token"], "launch_us": res["launch_us"],
                     "stream_read_GBs": stream_read_gbs(q)},
        "cpu_baseline": cpu,
        "variants": results,
        "e128": e128,
        "layer": layer,
        "attn": attn,
        "batch": batch,
        "requant": requant,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
