"""moe_decode_layer_noalloc (the layer call that allocates nothing: its
intermediates live in the library's static per-GPU scratch array) against
moe_decode_layer with a caller-owned workspace, through the C ABI: every
output and intermediate bit for bit, on calls in a row whose shapes shrink
and grow again (the array keeps the last call's contents), and a shape whose
intermediates exceed the array is refused."""
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


def _io(cfg, t, norm):
    H, E, k, F, Fs = cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs
    def z(*s, dt=torch.float32):
        if dt == torch.int32:
            return torch.full(s, -7, dtype=dt, device="cuda")
        return torch.zeros(*s, dtype=dt, device="cuda")
    io = {"routed_out": z(H, dt=torch.bfloat16), "xn": z(H), "xq": z(H // 32 * 36, dt=torch.uint8),
          "logits": z(E), "ids": z(k, dt=torch.int32), "weights": z(k), "h": z(k, F)}
    if Fs:
        io.update(shared_out=z(H, dt=torch.bfloat16), shared_gate=z(1), hs=z(Fs))
    ti = wl.token_inputs(cfg, t, "cuda")
    if norm:
        pv = wl.prev_outputs(cfg, t, "cuda")
        io.update(residual=ti["residual"], routed_in=pv["routed_prev"], out_sum=z(H, dt=torch.bfloat16))
        if "shared_prev" in pv:
            io["shared_in"] = pv["shared_prev"]
    else:
        io["x"] = ti["x"]
    return io


OUTS = ("out_sum", "routed_out", "shared_out", "xn", "xq", "logits", "ids", "weights", "shared_gate", "h", "hs")


def _compare(q, name, kw, t):
    cfg = wl.variant(wl.CONFIGS[name], **kw)
    norm = 1 if cfg.norm else 0
    gu.banner(f"no-alloc layer call: {name} {kw} token {t}")
    W = wl.layer_weights(cfg, 0, "cuda")
    desc = q.make_desc(cfg.H, cfg.E, cfg.k, cfg.F, cfg.Fs, norm=norm, eps=cfg.eps)
    ws = q.alloc_workspace(desc)
    ref, got = _io(cfg, t, norm), _io(cfg, t, norm)
    for key in ("residual", "routed_in", "shared_in", "x"):
        if key in ref:
            got[key] = ref[key]
    q.moe_decode_layer(desc, W, ref, ws)
    q.moe_decode_layer_noalloc(desc, W, got)
    torch.cuda.synchronize()
    for key in OUTS:
        if key in ref:
            assert torch.equal(ref[key].view(torch.uint8), got[key].view(torch.uint8)), (name, key)


def test_noalloc_matches_workspace_call_on_calls_in_a_row(q):
    _compare(q, "layer", {}, 0)                                  # H 2048, 256 experts, top-8, shared Q4_K
    _compare(q, "tiny", {}, 1)                                   # then a smaller input: H 512, 32 experts, no norm
    _compare(q, "layer", dict(E=64), 2)                          # and larger again
    _compare(q, "e128", dict(layers=1), 3)                       # F 768, no shared expert, 2-input fold


def test_noalloc_refuses_shapes_beyond_the_array(q):
    desc = q.make_desc(2048, 256, 16, 4096, 0)
    W = q.LayerWeights(**{n: 0x10000 for n, _ in q.LayerWeights._fields_})
    io = q.LayerIO(residual=0x10000, out_sum=0x10000, routed_out=0x10000)
    import ctypes as C
    assert q._moe_decode_layer_noalloc(C.byref(desc), C.byref(W), C.byref(io), None) == -5
