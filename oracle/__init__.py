"""ctypes binding of the CPU oracle (oracle/libmoe_oracle.so).

TEST INFRASTRUCTURE ONLY.  Imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark; never by the product package.  All arrays
are numpy arrays on the host.  bf16 and fp16 values travel as uint16 bit
patterns, quantised blocks as uint8 bytes.
"""
import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("MOE_ORACLE_LIB") or os.path.join(HERE, "libmoe_oracle.so")

Q8_0, Q8_1, Q4_K, Q5_K = 8, 9, 12, 13
BLOCK_BYTES = {Q4_K: 144, Q5_K: 176, Q8_0: 34, Q8_1: 36}

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            from . import build as _b
            _b.build()
        _lib = C.CDLL(LIB_PATH)
        _declare(_lib)
    return _lib


P = C.c_void_p


class Desc(C.Structure):
    _fields_ = [("H", C.c_int), ("E", C.c_int), ("k", C.c_int), ("F", C.c_int), ("Fs", C.c_int),
                ("gate_up_type", C.c_int), ("down_type", C.c_int), ("shared_type", C.c_int),
                ("norm", C.c_int), ("eps", C.c_float)]


class Weights(C.Structure):
    _fields_ = [(n, P) for n in ("norm_w", "router_w", "shared_gate_w", "gate", "up", "down",
                                 "sgate", "sup", "sdown")]


_OUT_FIELDS = ("out_sum", "xn", "xq", "logits", "z", "shared_gate", "ids", "weights", "h", "hs",
               "y", "ys", "routed", "shared", "routed_exact", "shared_exact")


class LayerOut(C.Structure):
    _fields_ = [(n, P) for n in _OUT_FIELDS]


def _declare(L):
    L.orc_f32_to_bf16.argtypes = [C.c_float]; L.orc_f32_to_bf16.restype = C.c_uint16
    L.orc_f32_to_f16.argtypes = [C.c_float]; L.orc_f32_to_f16.restype = C.c_uint16
    L.orc_bf16_to_f64.argtypes = [C.c_uint16]; L.orc_bf16_to_f64.restype = C.c_double
    L.orc_f16_to_f64.argtypes = [C.c_uint16]; L.orc_f16_to_f64.restype = C.c_double
    for n in ("orc_decode_q4k", "orc_decode_q5k", "orc_decode_q8_0"):
        getattr(L, n).argtypes = [P, P]; getattr(L, n).restype = None
    L.orc_decode_q8_1.argtypes = [P, P, P]; L.orc_decode_q8_1.restype = None
    L.orc_kquant_scales.argtypes = [P, P, P]; L.orc_kquant_scales.restype = None
    L.orc_quantize_q8_1.argtypes = [P, C.c_int, P]; L.orc_quantize_q8_1.restype = None
    L.orc_subblock_dots.argtypes = [P, C.c_int, C.c_int, P, P]; L.orc_subblock_dots.restype = C.c_int
    L.orc_row_dot.argtypes = [P, C.c_int, C.c_int, P]; L.orc_row_dot.restype = C.c_double
    L.orc_add_rmsnorm.argtypes = [P, P, P, P, C.c_int, C.c_float, P, P, P]; L.orc_add_rmsnorm.restype = None
    L.orc_router.argtypes = [P, P, C.c_int, C.c_int, P]; L.orc_router.restype = None
    L.orc_topk.argtypes = [P, C.c_int, C.c_int, P]; L.orc_topk.restype = None
    L.orc_softmax_selected.argtypes = [P, P, C.c_int, P]; L.orc_softmax_selected.restype = None
    L.orc_row_bytes.argtypes = [C.c_int, C.c_int]; L.orc_row_bytes.restype = C.c_long
    L.orc_pad_k.argtypes = [C.c_int, C.c_int]; L.orc_pad_k.restype = C.c_int
    L.orc_router_topk.argtypes = [P, P, P, P, P, P, P, P]; L.orc_router_topk.restype = None
    L.orc_expert_ffn.argtypes = [P, P, P, P, P, C.c_float, P]; L.orc_expert_ffn.restype = None
    L.orc_moe_layer.argtypes = [P, P, P, P, P, P, P]; L.orc_moe_layer.restype = C.c_int
    L.orc_moe_layer_sel.argtypes = [P, P, P, P, P, P, P, P]; L.orc_moe_layer_sel.restype = C.c_int
    L.orc_moe_stack.argtypes = [P, P, C.c_int, P, P, P, P, P, P, P]; L.orc_moe_stack.restype = C.c_int
    L.orc_num_threads.argtypes = []; L.orc_num_threads.restype = C.c_int
    L.orc_quantize_q4k.argtypes = [P, P]; L.orc_quantize_q4k.restype = None
    L.orc_requant_q4k.argtypes = [P, C.c_int, C.c_int, C.c_int, P]; L.orc_requant_q4k.restype = C.c_int
    L.orc_set_threads.argtypes = [C.c_int]; L.orc_set_threads.restype = None
    L.orc_moe_layer_batch.argtypes = [P, P, C.c_int, P, P, P, P, P]
    L.orc_moe_layer_batch.restype = C.c_int


def _p(a):
    """Pointer of a C-contiguous numpy array (None passes NULL)."""
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "oracle needs C-contiguous numpy arrays"
    return a.ctypes.data


def _u8(a):
    return np.ascontiguousarray(a, dtype=np.uint8)


# ---------------------------------------------------------------- scalars
def f32_to_bf16(x):
    L = lib()
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([L.orc_f32_to_bf16(float(v)) for v in x], dtype=np.uint16)


def f32_to_f16(x):
    L = lib()
    x = np.asarray(x, dtype=np.float32).ravel()
    return np.array([L.orc_f32_to_f16(C.c_float(v)) for v in x], dtype=np.uint16)


def bf16_to_f64(h):
    L = lib()
    return np.array([L.orc_bf16_to_f64(int(v)) for v in np.asarray(h, dtype=np.uint16).ravel()])


def f16_to_f64(h):
    L = lib()
    return np.array([L.orc_f16_to_f64(int(v)) for v in np.asarray(h, dtype=np.uint16).ravel()])


# ---------------------------------------------------------------- blocks
def decode(blocks, typ):
    """Decode a flat byte array of whole blocks of `typ` into fp64 values."""
    L = lib()
    b = _u8(blocks).ravel()
    nb = BLOCK_BYTES[typ]
    assert b.size % nb == 0
    n = b.size // nb
    per = 256 if typ in (Q4_K, Q5_K) else 32
    out = np.empty(n * per, dtype=np.float64)
    fn = {Q4_K: L.orc_decode_q4k, Q5_K: L.orc_decode_q5k, Q8_0: L.orc_decode_q8_0}.get(typ)
    for i in range(n):
        blk = b[i * nb:(i + 1) * nb]
        o = out[i * per:(i + 1) * per]
        if typ == Q8_1:
            L.orc_decode_q8_1(_p(blk), _p(o), None)
        else:
            fn(_p(blk), _p(o))
    return out


def q81_sums(blocks):
    """The stored s field of each Q8_1 block (fp64)."""
    L = lib()
    b = _u8(blocks).ravel()
    n = b.size // 36
    out = np.empty(n)
    tmp = np.empty(32)
    s = C.c_double()
    for i in range(n):
        blk = b[i * 36:(i + 1) * 36]
        L.orc_decode_q8_1(_p(blk), _p(tmp), C.byref(s))
        out[i] = s.value
    return out


def kquant_scales(blk):
    L = lib()
    sc = np.zeros(8, dtype=np.int32)
    m = np.zeros(8, dtype=np.int32)
    L.orc_kquant_scales(_p(_u8(blk)), _p(sc), _p(m))
    return sc, m


def quantize_q8_1(x):
    L = lib()
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    assert x.size % 32 == 0
    out = np.zeros(x.size // 32 * 36, dtype=np.uint8)
    L.orc_quantize_q8_1(_p(x), x.size, _p(out))
    return out


def quantize_q4k(x):
    """fp32 [..., K] (K % 256 == 0) -> Q4_K bytes, one call per superblock."""
    L = lib()
    x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1, 256)
    out = np.zeros(x.shape[0] * 144, dtype=np.uint8)
    for i in range(x.shape[0]):
        L.orc_quantize_q4k(_p(x[i]), _p(out[144 * i:]))
    return out


def requant_q4k(src, src_type, n_rows, K):
    """rows of K elements of src_type (Q8_0 / Q5_K / Q4_K) -> Q4_K rows (bytes)."""
    L = lib()
    src = _u8(src)
    out = np.zeros(n_rows * (K // 256) * 144, dtype=np.uint8)
    rc = L.orc_requant_q4k(_p(src), int(src_type), int(n_rows), int(K), _p(out))
    assert rc == 0, rc
    return out


def subblock_dots(row, typ, K, xq):
    L = lib()
    out = np.zeros(K // 32, dtype=np.int32)
    rc = L.orc_subblock_dots(_p(_u8(row)), typ, K, _p(_u8(xq)), _p(out))
    assert rc == 0
    return out


def row_dot(row, typ, K, xq):
    return lib().orc_row_dot(_p(_u8(row)), typ, K, _p(_u8(xq)))


def row_bytes(typ, K):
    return lib().orc_row_bytes(typ, K)


def pad_k(typ, K):
    return lib().orc_pad_k(typ, K)


# ---------------------------------------------------------------- steps
def add_rmsnorm(residual, routed, shared, w, eps):
    L = lib()
    residual = np.ascontiguousarray(residual, dtype=np.uint16)
    H = residual.size
    routed = None if routed is None else np.ascontiguousarray(routed, dtype=np.uint16)
    shared = None if shared is None else np.ascontiguousarray(shared, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    out_sum = np.zeros(H, dtype=np.uint16)
    xn = np.zeros(H, dtype=np.float32)
    xq = np.zeros(H // 32 * 36, dtype=np.uint8)
    L.orc_add_rmsnorm(_p(residual), _p(routed), _p(shared), _p(w), H, C.c_float(eps), _p(out_sum), _p(xn), _p(xq))
    return out_sum, xn, xq


def router(xn, W):
    L = lib()
    W = np.ascontiguousarray(W, dtype=np.float32)
    E, H = W.shape
    xn = np.ascontiguousarray(xn, dtype=np.float32)
    out = np.zeros(E, dtype=np.float32)
    L.orc_router(_p(xn), _p(W), E, H, _p(out))
    return out


def topk(logits, k):
    L = lib()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    ids = np.full(k, -1, dtype=np.int32)
    L.orc_topk(_p(logits), logits.size, k, _p(ids))
    return ids


def softmax_selected(logits, ids):
    L = lib()
    logits = np.ascontiguousarray(logits, dtype=np.float32)
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    w = np.zeros(ids.size, dtype=np.float32)
    L.orc_softmax_selected(_p(logits), _p(ids), ids.size, _p(w))
    return w


def num_threads():
    return lib().orc_num_threads()


def set_threads(n):
    lib().orc_set_threads(int(n))


# ---------------------------------------------------------------- layer
def make_desc(H, E, k, F, Fs, gate_up_type=Q4_K, down_type=Q4_K, shared_type=Q4_K, norm=1, eps=1e-6):
    return Desc(H, E, k, F, Fs, gate_up_type, down_type, shared_type, norm, eps)


class _Held:
    """Keeps numpy arrays alive while a ctypes struct points at them."""

    def __init__(self):
        self.arrays = []

    def hold(self, a, dtype):
        if a is None:
            return None
        a = np.ascontiguousarray(a, dtype=dtype)
        self.arrays.append(a)
        return a.ctypes.data


def make_weights(w, held):
    """w: dict with numpy arrays norm_w, router_w, shared_gate_w (fp32) and
    gate, up, down, sgate, sup, sdown (uint8 blocks); missing keys are NULL."""
    f32 = ("norm_w", "router_w", "shared_gate_w")
    vals = {}
    for n, _ in Weights._fields_:
        a = w.get(n)
        vals[n] = held.hold(a, np.float32 if n in f32 else np.uint8)
    return Weights(**vals)


def _alloc_out(desc):
    H, E, k, F, Fs = desc.H, desc.E, desc.k, desc.F, desc.Fs
    return {
        "out_sum": np.zeros(H, np.uint16), "xn": np.zeros(H, np.float32),
        "xq": np.zeros(H // 32 * 36, np.uint8), "logits": np.zeros(E, np.float32),
        "z": np.zeros(1, np.float32), "shared_gate": np.zeros(1, np.float32),
        "ids": np.zeros(k, np.int32), "weights": np.zeros(k, np.float32),
        "h": np.zeros(k * F, np.float32), "hs": np.zeros(max(Fs, 1), np.float32),
        "y": np.zeros(k * H, np.float32), "ys": np.zeros(H, np.float32),
        "routed": np.zeros(H, np.uint16), "shared": np.zeros(H, np.uint16),
        "routed_exact": np.zeros(H, np.float64), "shared_exact": np.zeros(H, np.float64),
    }


def moe_layer(desc, weights, residual=None, routed_prev=None, shared_prev=None, x=None, ids=None):
    """One layer for one token.  Returns a dict with every stored intermediate.
    ids (k experts in slot order) replaces the top-k selection (the near-tie
    rule of chained comparisons); the routing weights are then the softmax
    over those experts' logits."""
    L = lib()
    held = _Held()
    wst = make_weights(weights, held)
    out = _alloc_out(desc)
    lo = LayerOut(**{n: out[n].ctypes.data for n in _OUT_FIELDS})
    args = (C.byref(desc), C.byref(wst), held.hold(residual, np.uint16), held.hold(routed_prev, np.uint16),
            held.hold(shared_prev, np.uint16), held.hold(x, np.float32))
    if ids is None:
        rc = L.orc_moe_layer(*args, C.byref(lo))
    else:
        rc = L.orc_moe_layer_sel(*args, held.hold(ids, np.int32), C.byref(lo))
    if rc != 0:
        raise ValueError("oracle rejected the layer description or the selection")
    out["ids"] = out["ids"].copy()
    out["h"] = out["h"].reshape(desc.k, desc.F)
    out["y"] = out["y"].reshape(desc.k, desc.H)
    out["hs"] = out["hs"][:desc.Fs]
    return out


def router_topk(desc, weights, xn):
    L = lib()
    held = _Held()
    wst = make_weights(weights, held)
    xn = np.ascontiguousarray(xn, dtype=np.float32)
    logits = np.zeros(desc.E, np.float32)
    z = np.zeros(1, np.float32)
    ids = np.zeros(desc.k, np.int32)
    w = np.zeros(desc.k, np.float32)
    sg = np.zeros(1, np.float32)
    L.orc_router_topk(C.byref(desc), C.byref(wst), _p(xn), _p(logits), _p(z), _p(ids), _p(w), _p(sg))
    return dict(logits=logits, z=float(z[0]), ids=ids, weights=w, shared_gate=float(sg[0]))


def expert_ffn(desc, weights, xq, ids, wts, shared_gate):
    L = lib()
    held = _Held()
    wst = make_weights(weights, held)
    out = _alloc_out(desc)
    lo = LayerOut(**{n: out[n].ctypes.data for n in _OUT_FIELDS})
    L.orc_expert_ffn(C.byref(desc), C.byref(wst), held.hold(xq, np.uint8), held.hold(ids, np.int32),
                     held.hold(wts, np.float32), C.c_float(shared_gate), C.byref(lo))
    out["h"] = out["h"].reshape(desc.k, desc.F)
    out["y"] = out["y"].reshape(desc.k, desc.H)
    out["hs"] = out["hs"][:desc.Fs]
    return out


_BATCH_FIELDS = ("out_sum", "xn", "xq", "ids", "weights", "shared_gate", "group_size", "h", "hs", "y", "ys",
                 "routed", "shared", "routed_exact", "shared_exact")


class BatchOut(C.Structure):
    _fields_ = [(n, P) for n in _BATCH_FIELDS]


def moe_layer_batch(desc, weights, n_tok, residual=None, routed_prev=None, shared_prev=None, x=None):
    """One layer for n_tok tokens at once, experts grouped by the tokens that
    selected them; every group member gets the batch-1 integer path's result.
    Inputs are [n_tok][H] arrays; returns a dict of [n_tok][...] arrays."""
    L = lib()
    held = _Held()
    wst = make_weights(weights, held)
    H, k, F, Fs = desc.H, desc.k, desc.F, desc.Fs
    n = n_tok
    out = {
        "out_sum": np.zeros((n, H), np.uint16), "xn": np.zeros((n, H), np.float32),
        "xq": np.zeros((n, H // 32 * 36), np.uint8), "ids": np.zeros((n, k), np.int32),
        "weights": np.zeros((n, k), np.float32), "shared_gate": np.zeros(n, np.float32),
        "group_size": np.zeros((n, k), np.int32), "h": np.zeros((n, k, F), np.float32),
        "hs": np.zeros((n, max(Fs, 1)), np.float32), "y": np.zeros((n, k, H), np.float32),
        "ys": np.zeros((n, H), np.float32), "routed": np.zeros((n, H), np.uint16),
        "shared": np.zeros((n, H), np.uint16), "routed_exact": np.zeros((n, H), np.float64),
        "shared_exact": np.zeros((n, H), np.float64),
    }
    bo = BatchOut(**{f: out[f].ctypes.data for f in _BATCH_FIELDS})
    rc = L.orc_moe_layer_batch(C.byref(desc), C.byref(wst), n,
                               held.hold(residual, np.uint16), held.hold(routed_prev, np.uint16),
                               held.hold(shared_prev, np.uint16), held.hold(x, np.float32), C.byref(bo))
    if rc != 0:
        raise ValueError("oracle rejected the batch description")
    out["hs"] = out["hs"][:, :Fs]
    return out


def moe_stack(desc, layers, inp, per_layer=False, attn=None):
    """L-layer stack for one token; layers is a list of weight dicts; attn
    ([L][H] bf16 bits or None) is each layer's attention-block output."""
    L = lib()
    held = _Held()
    nl = len(layers)
    arr = (Weights * nl)(*[make_weights(w, held) for w in layers])
    inp = np.ascontiguousarray(inp, dtype=np.uint16)
    out = np.zeros(desc.H, np.uint16)
    ids = np.zeros((nl, desc.k), np.int32) if per_layer else None
    rt = np.zeros((nl, desc.H), np.uint16) if per_layer else None
    sh = np.zeros((nl, desc.H), np.uint16) if per_layer else None
    rs = np.zeros((nl, desc.H), np.uint16) if per_layer else None
    at = None if attn is None else np.ascontiguousarray(attn, dtype=np.uint16)
    rc = L.orc_moe_stack(C.byref(desc), arr, nl, _p(inp), _p(at), _p(out), _p(ids), _p(rt), _p(sh), _p(rs))
    if rc != 0:
        raise ValueError("oracle rejected the stack description")
    if per_layer:
        return out, dict(ids=ids, routed=rt, shared=sh, resid=rs)
    return out
