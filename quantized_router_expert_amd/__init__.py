"""Python binding of the gfx950 MoE decode library (libmoe_decode.so).

Argument marshalling only: torch tensors on the GPU are passed as device
pointers, the current torch stream as the HIP stream, and every computation
runs in the library's HIP kernels.  Importing this package loads the in-tree
shared library and raises if it is missing; there is no other code path.
The entry points keep the C names; each returns the C status and raises
MoeError on a non-zero status.
"""
import ctypes as C
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MOE_DECODE_LIB names another build of the same library (e.g. to compare two builds)
LIB_PATH = os.environ.get("MOE_DECODE_LIB") or os.path.join(HERE, "libmoe_decode.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built: run quantized_router_expert_amd/build.py (or __graft_entry__.build())")
_lib = C.CDLL(LIB_PATH)

Q8_0, Q8_1, Q4_K, Q5_K = 8, 9, 12, 13
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q8_0: 34, Q8_1: 36}
BLOCK_ELEMS = {Q4_K: 256, Q5_K: 256, Q8_0: 32, Q8_1: 32}
MOE_STACK_AUTO, MOE_STACK_KERNELS, MOE_STACK_PERSISTENT, MOE_STACK_COOPERATIVE = 0, 1, 2, 3
STATUS = {0: "MOE_OK", -1: "MOE_ERR_NULL", -2: "MOE_ERR_SHAPE", -3: "MOE_ERR_TYPE", -4: "MOE_ERR_ALIGN",
          -5: "MOE_ERR_WORKSPACE", -6: "MOE_ERR_HIP", -7: "MOE_ERR_UNSUPPORTED", -8: "MOE_ERR_NOT_BOUND"}


class MoeError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({moe_status_string(status)})")


P = C.c_void_p


class LayerDesc(C.Structure):
    _fields_ = [("hidden", C.c_int), ("n_experts", C.c_int), ("top_k", C.c_int), ("ffn", C.c_int),
                ("shared_ffn", C.c_int), ("gate_up_type", C.c_int), ("down_type", C.c_int),
                ("shared_type", C.c_int), ("norm", C.c_int), ("eps", C.c_float)]


class LayerWeights(C.Structure):
    _fields_ = [(n, P) for n in ("norm_w", "router_w", "shared_gate_w", "gate", "up", "down",
                                 "shared_gate", "shared_up", "shared_down")]


class StackIO(C.Structure):
    _fields_ = [("input", P), ("output", P), ("ids", P), ("resid", P), ("routed", P), ("shared", P),
                ("attn", P), ("trace", C.c_int)]


class LayerIO(C.Structure):
    _fields_ = [(n, P) for n in ("residual", "routed_in", "shared_in", "x", "out_sum", "routed_out", "shared_out",
                                 "xn", "xq", "logits", "ids", "weights", "shared_gate", "h", "hs")]


def _sig(name, res, *args):
    f = getattr(_lib, name)
    f.restype = res
    f.argtypes = list(args)
    return f


_moe_status_string = _sig("moe_status_string", C.c_char_p, C.c_int)
_moe_workspace_size = _sig("moe_workspace_size", C.c_size_t, C.POINTER(LayerDesc), C.c_int)
_moe_workspace_init = _sig("moe_workspace_init", C.c_int, P, C.c_size_t, P)
_add_rmsnorm3 = _sig("add_rmsnorm3", C.c_int, P, P, P, P, C.c_int, C.c_int, C.c_float, P, P, P, P)
_add_rmsnorm2_q8 = _sig("add_rmsnorm2_q8", C.c_int, P, P, P, C.c_int, C.c_int, C.c_float, P, P, P, P)
_router_topk = _sig("router_topk", C.c_int, P, P, P, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P, P, C.c_size_t, P)
_expert_ffn_q4k = _sig("expert_ffn_q4k", C.c_int, C.POINTER(LayerDesc), C.POINTER(LayerWeights), P, P, P, P, C.c_int,
                       P, P, P, P, P, C.c_size_t, P)
_moe_decode_layer = _sig("moe_decode_layer", C.c_int, C.POINTER(LayerDesc), C.POINTER(LayerWeights),
                         C.POINTER(LayerIO), P, C.c_size_t, P)
_moe_stack_bind = _sig("moe_stack_bind", C.c_int, C.POINTER(LayerDesc), C.POINTER(LayerWeights), C.c_int, P,
                       C.c_size_t, P)
_moe_decode_stack = _sig("moe_decode_stack", C.c_int, C.POINTER(LayerDesc), C.POINTER(LayerWeights), C.c_int,
                         C.POINTER(StackIO), C.c_int, P, C.c_size_t, P)
_moe_decode_layer_noalloc = _sig("moe_decode_layer_noalloc", C.c_int, C.POINTER(LayerDesc), C.POINTER(LayerWeights),
                                 C.POINTER(LayerIO), P)
_moe_batch_workspace_size = _sig("moe_batch_workspace_size", C.c_size_t, C.POINTER(LayerDesc), C.c_int)
_expert_ffn_grouped = _sig("expert_ffn_grouped", C.c_int, C.POINTER(LayerDesc), C.POINTER(LayerWeights), P, P, P, P, P,
                           C.c_int, C.c_int, P, P, P, P, P, C.c_size_t, P)
_moe_decode_layer_batch = _sig("moe_decode_layer_batch", C.c_int, C.POINTER(LayerDesc), C.POINTER(LayerWeights),
                               C.POINTER(LayerIO), C.c_int, C.c_int, P, C.c_size_t, P)
_moe_tune_group_min = _sig("moe_tune_group_min", C.c_int, C.POINTER(LayerDesc), C.POINTER(LayerWeights),
                           C.POINTER(LayerIO), C.c_int, C.POINTER(C.c_int), C.c_int, C.c_int, P, C.c_size_t, P,
                           C.POINTER(C.c_int), C.POINTER(C.c_float))
_moe_stack_status_offset = _sig("moe_stack_status_offset", C.c_size_t, C.POINTER(LayerDesc), C.c_int)
_moe_stack_kernel_shape = _sig("moe_stack_kernel_shape", C.c_int, C.POINTER(LayerDesc))
_moe_stack_trace_offset = _sig("moe_stack_trace_offset", C.c_size_t, C.POINTER(LayerDesc), C.c_int)
_moe_test_subblock_dots = _sig("moe_test_subblock_dots", C.c_int, P, C.c_int, C.c_int, C.c_int, P, P, P)
_moe_test_quantize_q81 = _sig("moe_test_quantize_q81", C.c_int, P, C.c_int, P, P)
_moe_stream_read = _sig("moe_stream_read", C.c_int, P, C.c_size_t, P, C.c_int, P)
_moe_test_stack_select = _sig("moe_test_stack_select", C.c_int, P, C.c_int, C.c_int, C.c_int, C.c_int, P, P, P, P)
_moe_requant_q4k = _sig("moe_requant_q4k", C.c_int, P, C.c_int, C.c_int, C.c_int, P, P)

EXPORTS = ("add_rmsnorm3", "router_topk", "expert_ffn_q4k", "moe_decode_layer", "moe_stack_bind",
           "moe_decode_stack", "moe_workspace_size", "moe_workspace_init", "moe_status_string",
           "moe_stack_status_offset", "moe_stack_trace_offset", "moe_test_subblock_dots", "moe_test_quantize_q81", "moe_stream_read", "moe_requant_q4k",
           "moe_batch_workspace_size", "expert_ffn_grouped", "moe_decode_layer_batch", "moe_test_stack_select",
           "moe_decode_layer_noalloc", "add_rmsnorm2_q8", "moe_stack_kernel_shape", "moe_tune_group_min")
MAX_BATCH = 64
MAX_GROUP_MIN = 16


# ---------------------------------------------------------------- marshalling helpers
def ptr(t):
    """Device pointer of a CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def stream_handle(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def _check(fn, rc):
    if rc != 0:
        raise MoeError(fn, rc)
    return rc


def make_desc(hidden, n_experts, top_k, ffn, shared_ffn, gate_up_type=Q4_K, down_type=Q4_K, shared_type=Q4_K,
              norm=1, eps=1e-6):
    return LayerDesc(hidden, n_experts, top_k, ffn, shared_ffn, gate_up_type, down_type, shared_type, norm, eps)


def make_weights(w):
    """dict of CUDA tensors (keys as in moe_layer_weights, generator names accepted) -> LayerWeights."""
    alias = {"sgate": "shared_gate", "sup": "shared_up", "sdown": "shared_down"}
    vals = {}
    for k, v in w.items():
        if k.startswith("_"):
            continue
        vals[alias.get(k, k)] = ptr(v)
    return LayerWeights(**{n: vals.get(n) for n, _ in LayerWeights._fields_})


# ---------------------------------------------------------------- entry points
def moe_status_string(status):
    return _moe_status_string(status).decode()


def moe_workspace_size(desc, n_layers=0):
    return _moe_workspace_size(C.byref(desc), n_layers)


def moe_workspace_init(ws, stream=None):
    return _check("moe_workspace_init", _moe_workspace_init(ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)))


def alloc_workspace(desc, n_layers=0, extra=0, device="cuda"):
    """A zero-initialised, 256-byte aligned workspace tensor for `desc`."""
    n = moe_workspace_size(desc, n_layers) + extra
    if n == 0:
        raise MoeError("moe_workspace_size", -2)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    moe_workspace_init(ws)
    return ws


def add_rmsnorm3(residual, routed, shared, norm_w, hidden, n_tok, eps, out_sum, xn=None, xq=None, stream=None):
    return _check("add_rmsnorm3", _add_rmsnorm3(ptr(residual), ptr(routed), ptr(shared), ptr(norm_w), hidden, n_tok,
                                                eps, ptr(out_sum), ptr(xn), ptr(xq), stream_handle(stream)))


def add_rmsnorm2_q8(residual, attn_out, norm_w, hidden, n_tok, eps, out_sum, xn=None, xq=None, stream=None):
    return _check("add_rmsnorm2_q8", _add_rmsnorm2_q8(ptr(residual), ptr(attn_out), ptr(norm_w), hidden, n_tok, eps,
                                                      ptr(out_sum), ptr(xn), ptr(xq), stream_handle(stream)))


def router_topk(xn, w_router, w_shared_gate, n_tok, hidden, n_experts, top_k, logits, ids, weights, shared_gate_out,
                ws, stream=None):
    return _check("router_topk", _router_topk(ptr(xn), ptr(w_router), ptr(w_shared_gate), n_tok, hidden, n_experts,
                                              top_k, ptr(logits), ptr(ids), ptr(weights), ptr(shared_gate_out),
                                              ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)))


def router_ws_bytes(n_tok, n_experts):
    return 16384 + ((4 * n_tok * (n_experts + 1) + 255) // 256) * 256


def expert_ffn_q4k(desc, weights, xq, ids, wts, shared_gate, n_tok, routed_out, shared_out, h, hs, ws, stream=None):
    lw = weights if isinstance(weights, LayerWeights) else make_weights(weights)
    return _check("expert_ffn_q4k", _expert_ffn_q4k(C.byref(desc), C.byref(lw), ptr(xq), ptr(ids), ptr(wts),
                                                    ptr(shared_gate), n_tok, ptr(routed_out), ptr(shared_out),
                                                    ptr(h), ptr(hs), ptr(ws), ws.numel() * ws.element_size(),
                                                    stream_handle(stream)))


def moe_decode_layer(desc, weights, io, ws, stream=None):
    """io: dict of CUDA tensors keyed by the moe_layer_io field names."""
    lw = weights if isinstance(weights, LayerWeights) else make_weights(weights)
    lio = LayerIO(**{n: ptr(io.get(n)) for n, _ in LayerIO._fields_})
    return _check("moe_decode_layer", _moe_decode_layer(C.byref(desc), C.byref(lw), C.byref(lio), ptr(ws),
                                                        ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_decode_layer_noalloc(desc, weights, io, stream=None):
    """moe_decode_layer with the library's static scratch array instead of a workspace."""
    lw = weights if isinstance(weights, LayerWeights) else make_weights(weights)
    lio = LayerIO(**{n: ptr(io.get(n)) for n, _ in LayerIO._fields_})
    return _check("moe_decode_layer_noalloc", _moe_decode_layer_noalloc(C.byref(desc), C.byref(lw), C.byref(lio),
                                                                        stream_handle(stream)))


def moe_batch_workspace_size(desc, n_tok):
    return _moe_batch_workspace_size(C.byref(desc), n_tok)


def alloc_batch_workspace(desc, n_tok, device="cuda"):
    """A zero-initialised, 256-byte aligned workspace for the grouped path."""
    n = moe_batch_workspace_size(desc, n_tok)
    if n == 0:
        raise MoeError("moe_batch_workspace_size", -2)
    ws = torch.empty(n + 256, dtype=torch.uint8, device=device)
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    moe_workspace_init(ws)
    return ws


def expert_ffn_grouped(desc, weights, xn, xq, ids, wts, shared_gate, n_tok, group_min, routed_out, shared_out,
                       h, hs, ws, stream=None):
    lw = weights if isinstance(weights, LayerWeights) else make_weights(weights)
    return _check("expert_ffn_grouped", _expert_ffn_grouped(C.byref(desc), C.byref(lw), ptr(xn), ptr(xq), ptr(ids),
                                                            ptr(wts), ptr(shared_gate), n_tok, group_min,
                                                            ptr(routed_out), ptr(shared_out), ptr(h), ptr(hs),
                                                            ptr(ws), ws.numel() * ws.element_size(),
                                                            stream_handle(stream)))


def moe_decode_layer_batch(desc, weights, io, n_tok, group_min, ws, stream=None):
    """io: dict of CUDA tensors ([n_tok][...]) keyed by the moe_layer_io field names."""
    lw = weights if isinstance(weights, LayerWeights) else make_weights(weights)
    lio = LayerIO(**{n: ptr(io.get(n)) for n, _ in LayerIO._fields_})
    return _check("moe_decode_layer_batch", _moe_decode_layer_batch(C.byref(desc), C.byref(lw), C.byref(lio), n_tok,
                                                                    group_min, ptr(ws), ws.numel() * ws.element_size(),
                                                                    stream_handle(stream)))


def tune_group_min(desc, weights, io, n_tok, ws, candidates=(4, 6, 9, 12, 16), reps=5, stream=None):
    """(best group_min, its mean us per call) measured on this device; io's outputs are overwritten."""
    lw = weights if isinstance(weights, LayerWeights) else make_weights(weights)
    lio = LayerIO(**{n: ptr(io.get(n)) for n, _ in LayerIO._fields_})
    cand = (C.c_int * len(candidates))(*candidates)
    best, us = C.c_int(0), C.c_float(0.0)
    _check("moe_tune_group_min", _moe_tune_group_min(C.byref(desc), C.byref(lw), C.byref(lio), n_tok, cand,
                                                     len(candidates), reps, ptr(ws), ws.numel() * ws.element_size(),
                                                     stream_handle(stream), C.byref(best), C.byref(us)))
    return best.value, us.value


def _layer_array(layers):
    arr = (LayerWeights * len(layers))()
    for i, w in enumerate(layers):
        arr[i] = w if isinstance(w, LayerWeights) else make_weights(w)
    return arr


def moe_stack_bind(desc, layers, ws, stream=None):
    arr = _layer_array(layers)
    return _check("moe_stack_bind", _moe_stack_bind(C.byref(desc), arr, len(layers), ptr(ws),
                                                    ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_decode_stack(desc, layers, inp, out, ids_per_layer=None, resid_per_layer=None, mode=MOE_STACK_AUTO, ws=None,
                     stream=None, layer_array=None, routed_per_layer=None, shared_per_layer=None, trace=0, attn=None):
    arr = layer_array if layer_array is not None else _layer_array(layers)
    n = len(arr)
    io = StackIO(ptr(inp), ptr(out), ptr(ids_per_layer), ptr(resid_per_layer), ptr(routed_per_layer),
                 ptr(shared_per_layer), ptr(attn), int(trace))
    return _check("moe_decode_stack", _moe_decode_stack(C.byref(desc), arr, n, C.byref(io), mode, ptr(ws),
                                                        ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_stack_status_offset(desc, n_layers):
    return _moe_stack_status_offset(C.byref(desc), n_layers)


def stack_status(desc, n_layers, ws):
    """The persistent stack's status word (reads the device workspace; synchronises)."""
    off = moe_stack_status_offset(desc, n_layers)
    if off == 0:
        raise MoeError("moe_stack_status_offset", -7)
    return int(ws[off:off + 4].view(torch.int32).item())


def stack_stop_detail(desc, n_layers, ws):
    """After a stopped persistent launch (status 1): (layer, check) of the stop."""
    off = moe_stack_status_offset(desc, n_layers)
    if off == 0:
        raise MoeError("moe_stack_status_offset", -7)
    v = int(ws[off + 4:off + 8].view(torch.int32).item())
    return v >> 8, v & 0xff


def moe_stack_kernel_shape(desc):
    """0 = generic persistent instance, n >= 1 = compile-time shape n, -1 = none."""
    return _moe_stack_kernel_shape(C.byref(desc))


def moe_stack_trace_offset(desc, n_layers):
    return _moe_stack_trace_offset(C.byref(desc), n_layers)


TRACE_SLOTS = 12


def stack_trace(desc, n_layers, ws):
    """Per-layer phase timestamps (microseconds from workgroup 0's layer start)
    of the last persistent launch, as a [min(L, 64), 10] float tensor, and the
    shader clock in MHz over those layers (reads the workspace)."""
    off = moe_stack_trace_offset(desc, n_layers)
    if off == 0:
        raise MoeError("moe_stack_trace_offset", -7)
    n = min(n_layers, 64)
    t = ws[off:off + 8 * 64 * TRACE_SLOTS].view(torch.int64).view(64, TRACE_SLOTS)[:n].double().cpu()
    mhz = float(((t[:, 11] - t[:, 10]).sum() / ((t[:, 9] - t[:, 0]).sum() / 100.0)))
    return (t[:, :10] - t[:, :1]) / 100.0, mhz


BLOCK_EVENTS = 16
TRACE_MAX_G = 256


def stack_block_trace(desc, n_layers, ws):
    """Per-workgroup event times of the last persistent launch, in microseconds
    of the device wall clock, as a [min(L, 64), 256, 16] float tensor (written
    only by launches made with trace=1):
    0 layer start, 1 previous outputs received, 2 fixed weights landed,
    3 router rows stored, 4 shared h stored, 5 experts known, 6 routed gate/up
    rows landed, 7 routed h stored, 8 down inputs quantised, 9 down rows landed,
    10 layer outputs stored, 11 input normalised, 12 input quantised, 13 logits
    received, 14 every h received, 15 down rows queued."""
    off = moe_stack_trace_offset(desc, n_layers)
    if off == 0:
        raise MoeError("moe_stack_trace_offset", -7)
    off += 8 * 64 * TRACE_SLOTS
    n = min(n_layers, 64)
    t = ws[off:off + 8 * 64 * TRACE_MAX_G * BLOCK_EVENTS].view(torch.int64).view(64, TRACE_MAX_G, BLOCK_EVENTS)
    return t[:n].double().cpu() / 100.0


def layer_array(layers):
    """Pre-marshalled host array of layer weight pointers (reuse across calls)."""
    return _layer_array(layers)


def moe_requant_q4k(src, src_type, n_rows, K, dst, stream=None):
    return _check("moe_requant_q4k", _moe_requant_q4k(ptr(src), src_type, n_rows, K, ptr(dst), stream_handle(stream)))


def moe_stream_read(p, n_bytes, out, blocks, stream=None):
    return _check("moe_stream_read", _moe_stream_read(ptr(p), n_bytes, ptr(out), blocks, stream_handle(stream)))


def moe_test_quantize_q81(x, n, xq, stream=None):
    return _check("moe_test_quantize_q81", _moe_test_quantize_q81(ptr(x), n, ptr(xq), stream_handle(stream)))


def moe_test_stack_select(logits, n_sets, n_experts, top_k, with_gate, ids, weights, gate=None, stream=None):
    return _check("moe_test_stack_select", _moe_test_stack_select(ptr(logits), n_sets, n_experts, top_k, int(with_gate),
                                                                  ptr(ids), ptr(weights), ptr(gate),
                                                                  stream_handle(stream)))


def moe_test_subblock_dots(rows, typ, K, n_rows, xq, out, stream=None):
    return _check("moe_test_subblock_dots", _moe_test_subblock_dots(ptr(rows), typ, K, n_rows, ptr(xq), ptr(out),
                                                                    stream_handle(stream)))


def raw_call(name, *args):
    """Call an exported C function with raw ctypes-compatible arguments (tests of the
    argument validation use this to pass NULL/misaligned pointers)."""
    return getattr(_lib, name)(*args)
