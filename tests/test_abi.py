"""The C-ABI library loads, exports every function include/moe_decode.h
declares, and rejects invalid arguments with the documented codes on the
host, before anything is enqueued (these calls need no GPU)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_decode.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s+\*?([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("add_rmsnorm3", "add_rmsnorm2_q8", "router_topk", "expert_ffn_q4k", "moe_decode_layer", "moe_decode_stack",
              "moe_stack_bind", "moe_workspace_size", "moe_workspace_init", "moe_status_string",
              "moe_test_subblock_dots", "moe_test_quantize_q81"):
        assert n in names, n


def test_library_exports_every_declared_symbol():
    import quantized_router_expert_amd as q
    lib = C.CDLL(q.LIB_PATH)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in moe_decode.h but not exported"
    assert set(q.EXPORTS) <= set(declared_functions())


@pytest.fixture(scope="module")
def q():
    import quantized_router_expert_amd as q
    return q


def _desc(q, **kw):
    d = dict(hidden=2048, n_experts=256, top_k=8, ffn=512, shared_ffn=512)
    d.update(kw)
    return q.make_desc(**d)


def test_status_strings(q):
    assert q.moe_status_string(0) == "ok"
    for s in range(-1, -9, -1):
        assert q.moe_status_string(s) != "unknown status"


def test_workspace_size(q):
    assert q.moe_workspace_size(_desc(q)) > 0
    assert q.moe_workspace_size(_desc(q), 40) > q.moe_workspace_size(_desc(q), 0)
    assert q.moe_workspace_size(_desc(q, hidden=100)) == 0          # invalid desc -> 0
    assert q.moe_workspace_size(_desc(q, top_k=300)) == 0


FAKE = 0x10000       # 256-aligned fake device address: never dereferenced on these paths
ODD = 0x10001


def test_add_rmsnorm3_validation(q):
    f = q._add_rmsnorm3
    ok = dict(res=FAKE, rt=None, sh=None, w=FAKE, H=2048, n=1, eps=1e-6, out=FAKE, xn=None, xq=None)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return f(a["res"], a["rt"], a["sh"], a["w"], a["H"], a["n"], a["eps"], a["out"], a["xn"], a["xq"], None)

    assert call(res=None) == -1
    assert call(w=None) == -1
    assert call(out=None) == -1
    assert call(sh=FAKE, rt=None) == -1          # shared without routed
    assert call(H=100) == -2
    assert call(H=0) == -2
    assert call(H=16384) == -2
    assert call(n=0) == -2
    assert call(eps=-1.0) == -2
    assert call(eps=float("nan")) == -2
    assert call(res=ODD) == -4
    assert call(xq=FAKE + 2) == -4
    assert q._add_rmsnorm2_q8(FAKE, None, FAKE, 2048, 1, 1e-6, FAKE, None, None, None) == -1
    assert q._add_rmsnorm2_q8(FAKE, FAKE, FAKE, 100, 1, 1e-6, FAKE, None, None, None) == -2


def test_router_topk_validation(q):
    f = q._router_topk

    def call(xn=FAKE, W=FAKE, g=None, n=1, H=2048, E=256, k=8, lg=None, ids=FAKE, w=FAKE, sg=None, ws=FAKE,
             wsb=1 << 20):
        return f(xn, W, g, n, H, E, k, lg, ids, w, sg, ws, wsb, None)

    assert call(xn=None) == -1
    assert call(ids=None) == -1
    assert call(k=0) == -2
    assert call(k=9, E=8) == -2
    assert call(k=17, E=256) == -2
    assert call(E=2000) == -2
    assert call(H=1000) == -2
    assert call(n=5000) == -2
    assert call(xn=FAKE + 4) == -4               # float4 loads need 16-byte alignment
    assert call(ws=None) == -5
    assert call(wsb=1024) == -5
    assert call(ws=FAKE + 16) == -4


def test_expert_ffn_validation(q):
    d = _desc(q)
    good = q.LayerWeights(norm_w=FAKE, router_w=FAKE, shared_gate_w=FAKE, gate=FAKE, up=FAKE, down=FAKE,
                          shared_gate=FAKE, shared_up=FAKE, shared_down=FAKE)
    f = q._expert_ffn_q4k

    def call(desc=d, w=good, xq=FAKE, ids=FAKE, wts=FAKE, sg=FAKE, n=1, ro=FAKE, so=FAKE, ws=FAKE, wsb=1 << 24):
        return f(C.byref(desc), C.byref(w), xq, ids, wts, sg, n, ro, so, None, None, ws, wsb, None)

    assert call(xq=None) == -1
    assert call(sg=None) == -1                                    # shared expert needs the gate value
    assert call(n=2) == -7
    assert call(desc=_desc(q, gate_up_type=13)) == -3
    assert call(desc=_desc(q, down_type=8)) == -3
    assert call(desc=_desc(q, shared_type=13)) == -3
    assert call(desc=_desc(q, ffn=100)) == -2
    assert call(desc=_desc(q, shared_type=8, shared_ffn=128)) == -2  # Q8_0 rows must be whole 16-byte multiples
    bad = q.LayerWeights(**{n: FAKE for n, _ in q.LayerWeights._fields_})
    bad.gate = FAKE + 8
    assert call(w=bad) == -4
    nul = q.LayerWeights(**{n: FAKE for n, _ in q.LayerWeights._fields_})
    nul.down = None
    assert call(w=nul) == -1
    assert call(wsb=100) == -5


def test_layer_and_stack_validation(q):
    d = _desc(q)
    w = q.LayerWeights(**{n: FAKE for n, _ in q.LayerWeights._fields_})
    io = q.LayerIO(residual=FAKE, out_sum=FAKE, routed_out=FAKE, shared_out=FAKE)
    assert q._moe_decode_layer(C.byref(d), C.byref(w), None, FAKE, 1 << 24, None) == -1
    io2 = q.LayerIO(residual=None, out_sum=FAKE, routed_out=FAKE, shared_out=FAKE)
    assert q._moe_decode_layer(C.byref(d), C.byref(w), C.byref(io2), FAKE, 1 << 24, None) == -1
    assert q._moe_decode_layer(C.byref(d), C.byref(w), C.byref(io), FAKE, 16, None) == -5
    arr = (q.LayerWeights * 2)(w, w)
    sio = q.StackIO(input=FAKE, output=FAKE)
    big = q.moe_workspace_size(d, 2)
    ds = q._moe_decode_stack
    assert ds(C.byref(d), arr, 0, C.byref(sio), 0, FAKE, big, None) == -2
    assert ds(C.byref(d), arr, 2, C.byref(sio), 9, FAKE, big, None) == -2
    assert ds(C.byref(d), arr, 2, None, 0, FAKE, big, None) == -1
    assert ds(C.byref(d), arr, 2, C.byref(q.StackIO(input=None, output=FAKE)), 0, FAKE, big, None) == -1
    assert ds(C.byref(d), arr, 2, C.byref(q.StackIO(input=FAKE, output=FAKE, routed=FAKE + 1)), 0, FAKE, big,
              None) == -4
    assert ds(C.byref(d), arr, 2, C.byref(sio), 0, FAKE, big - 1, None) == -5
    d0 = _desc(q, norm=0)
    assert ds(C.byref(d0), arr, 2, C.byref(sio), 0, FAKE, big, None) == -7
    # the persistent kernel on a workspace that holds no bound stack: refused
    # on the host before anything is enqueued
    assert ds(C.byref(d), arr, 2, C.byref(sio), q.MOE_STACK_PERSISTENT, FAKE, big, None) == -8
    assert ds(C.byref(d), arr, 2, C.byref(sio), q.MOE_STACK_COOPERATIVE, FAKE, big, None) == -8
    assert ds(C.byref(d), arr, 2, C.byref(sio), 4, FAKE, big, None) == -2
    assert q._moe_stack_bind(C.byref(d), arr, 2, FAKE, 1024, None) == -5
    assert q._moe_test_subblock_dots(FAKE, 9, 256, 1, FAKE, FAKE, None) == -3
    assert q._moe_test_subblock_dots(FAKE, 12, 100, 1, FAKE, FAKE, None) == -2
    assert q._moe_test_quantize_q81(None, 32, FAKE, None) == -1
    assert q._moe_test_quantize_q81(FAKE, 48, FAKE, None) == -2
    assert q._moe_test_quantize_q81(FAKE + 4, 32, FAKE, None) == -4
    assert q._moe_requant_q4k(None, 13, 1, 256, FAKE, None) == -1
    assert q._moe_requant_q4k(FAKE, 9, 1, 256, FAKE, None) == -3
    assert q._moe_requant_q4k(FAKE, 13, 1, 300, FAKE, None) == -2
    assert q._moe_requant_q4k(FAKE, 13, 0, 256, FAKE, None) == -2
    assert q._moe_requant_q4k(FAKE + 8, 13, 1, 256, FAKE, None) == -4
    assert q._moe_requant_q4k(FAKE, 13, 1, 256, FAKE + 1, None) == -4
    assert q._moe_stream_read(None, 1024, FAKE, 8, None) == -1
    assert q._moe_stream_read(FAKE, 1000, FAKE, 8, None) == -2
    assert q._moe_stream_read(FAKE, 1024, FAKE, 0, None) == -2
    assert q._moe_stream_read(FAKE + 8, 1024, FAKE, 8, None) == -4
    sel = q._moe_test_stack_select
    assert sel(None, 1, 256, 8, 0, FAKE, FAKE, None, None) == -1
    assert sel(FAKE, 1, 256, 8, 1, FAKE, FAKE, None, None) == -1    # the gate output is needed
    assert sel(FAKE, 0, 256, 8, 0, FAKE, FAKE, None, None) == -2
    assert sel(FAKE, 1, 4, 8, 0, FAKE, FAKE, None, None) == -2      # k > E
    assert sel(FAKE, 1, 2048, 8, 0, FAKE, FAKE, None, None) == -2
    assert sel(FAKE, 1, 256, 17, 0, FAKE, FAKE, None, None) == -2
    assert sel(FAKE + 2, 1, 256, 8, 0, FAKE, FAKE, None, None) == -4
    na = q._moe_decode_layer_noalloc
    assert na(C.byref(d), C.byref(w), None, None) == -1
    assert na(C.byref(d), C.byref(w), C.byref(io2), None) == -1
    big = _desc(q, top_k=16, ffn=4096, shared_ffn=0)           # intermediates beyond the static array
    assert na(C.byref(big), C.byref(w), C.byref(io), None) == -5
    assert q._moe_workspace_init(None, 1024, None) == -5
    assert q._moe_workspace_init(FAKE + 8, 1024, None) == -4


def test_grouped_path_validation(q):
    d = _desc(q)
    w = q.LayerWeights(**{n: FAKE for n, _ in q.LayerWeights._fields_})
    f = q._expert_ffn_grouped
    need = q.moe_batch_workspace_size(d, 8)
    assert need > 0
    assert q.moe_batch_workspace_size(d, 0) == 0 and q.moe_batch_workspace_size(d, 65) == 0

    def call(xn=FAKE, xq=FAKE, ids=FAKE, wts=FAKE, sg=FAKE, n=8, gmin=4, ro=FAKE, so=FAKE, h=None, hs=None, ws=FAKE,
             wsb=need):
        return f(C.byref(d), C.byref(w), xn, xq, ids, wts, sg, n, gmin, ro, so, h, hs, ws, wsb, None)

    assert call(xn=None) == -1
    assert call(sg=None) == -1                   # the shared expert needs its gate values
    assert call(so=None) == -1
    assert call(n=0) == -2
    assert call(n=65) == -2
    assert call(gmin=0) == -2
    assert call(gmin=17) == -2
    assert call(xn=FAKE + 4) == -4               # the bf16 path reads xn 16 bytes at a time
    assert call(h=FAKE + 8) == -4
    assert call(wsb=need - 1) == -5
    io = q.LayerIO(residual=FAKE, out_sum=FAKE, routed_out=FAKE, shared_out=FAKE)
    g = q._moe_decode_layer_batch
    assert g(C.byref(d), C.byref(w), C.byref(io), 8, 4, FAKE, need - 1, None) == -5
    assert g(C.byref(d), C.byref(w), C.byref(io), 0, 4, FAKE, need, None) == -2
    assert g(C.byref(d), C.byref(w), C.byref(io), 8, 99, FAKE, need, None) == -2
    io2 = q.LayerIO(residual=FAKE, out_sum=FAKE, routed_out=FAKE, shared_out=None)
    assert g(C.byref(d), C.byref(w), C.byref(io2), 8, 4, FAKE, need, None) == -1


def test_tune_group_min_rejects_bad_arguments():
    """The group_min tuner validates its host arguments before any device call."""
    import quantized_router_expert_amd as q
    lib = C.CDLL(q.LIB_PATH)
    f = lib.moe_tune_group_min
    f.restype = C.c_int
    f.argtypes = [C.c_void_p] * 3 + [C.c_int, C.c_void_p, C.c_int, C.c_int, C.c_void_p, C.c_size_t, C.c_void_p,
                                     C.c_void_p, C.c_void_p]
    best = C.c_int(-1)
    cand = (C.c_int * 3)(4, 9, 16)
    assert f(None, None, None, 8, None, 3, 5, None, 0, None, C.byref(best), None) == -1
    assert f(None, None, None, 8, cand, 3, 5, None, 0, None, None, None) == -1
    assert f(None, None, None, 8, cand, 0, 5, None, 0, None, C.byref(best), None) == -2
    assert f(None, None, None, 8, cand, 3, 0, None, 0, None, C.byref(best), None) == -2
    assert f(None, None, None, 8, cand, 3, 101, None, 0, None, C.byref(best), None) == -2
    bad = (C.c_int * 2)(4, q.MAX_GROUP_MIN + 1)
    assert f(None, None, None, 8, bad, 2, 5, None, 0, None, C.byref(best), None) == -2
    assert best.value == -1


def test_header_compiles_as_plain_c(tmp_path):
    """The boundary is a C ABI: the public header compiles as C99 with warnings as errors."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use_header.c"
    src.write_text(f'#include "{HEADER}"\nint main(void) {{ return moe_status_string(0) == 0; }}\n')
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-c", str(src), "-o",
                        str(tmp_path / "use_header.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
