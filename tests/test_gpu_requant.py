"""Parity of the load-time requantisation to Q4_K (moe_requant_q4k) with the
oracle: the Q4_K bytes must be identical (every step of the quantiser is an
fp32 operation rounded to nearest, taken in the same order on both sides).

Small cases cover every source type, ragged row counts and the degenerate
sub-blocks (all zero, all positive, all negative, one value, signed zeros);
the full-size case requantises one layer's 256 routed down matrices (Q5_K,
2048 x 512 each) and one shared expert (Q8_0) and checks sampled superblocks.
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


def _x(n_rows, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n_rows * K // 32, 32)) * 0.02
    kind = rng.integers(0, 10, x.shape[0])
    x[kind == 1] = np.abs(x[kind == 1])
    x[kind == 2] = -np.abs(x[kind == 2])
    x[kind == 3] = 0.0
    x[kind == 4, 1:] = 0.0
    x[kind == 5] = -0.0
    x *= np.exp2(rng.integers(-6, 4, (x.shape[0] // 8, 1))).repeat(8, 0)
    return torch.from_numpy(x.astype(np.float32).reshape(n_rows, K))


def _run(q, src, src_type, n_rows, K, skew=0):
    """skew: bytes past a 16-byte boundary for dst (2: the library's
    superblock-per-wave kernel, which needs only 2-byte alignment; 0: the
    sub-block-per-lane kernel)."""
    n = n_rows * (K // 256) * 144
    buf = torch.zeros(n + 16, dtype=torch.uint8, device="cuda")
    dst = buf[skew:skew + n]
    q.moe_requant_q4k(src, src_type, n_rows, K, dst)
    torch.cuda.synchronize()
    return dst


@pytest.mark.parametrize("src_type", [wl.Q8_0, wl.Q5_K, wl.Q4_K])
@pytest.mark.parametrize("n_rows,K,skew", [(1, 256, 0), (37, 2048, 0), (5, 768, 0), (37, 2048, 2), (3, 256, 2)])
def test_requant_bit_exact(q, orc, src_type, n_rows, K, skew):
    gu.banner(f"requant to Q4_K from type {src_type}, {n_rows} x {K}, dst skew {skew}")
    src = wl.quantize(_x(n_rows, K, 100 * src_type + K + n_rows), src_type).numpy()
    got = gu.host(_run(q, gu.dev(src), src_type, n_rows, K, skew))
    ref = orc.requant_q4k(src, src_type, n_rows, K)
    bad = np.nonzero((got.reshape(-1, 144) != ref.reshape(-1, 144)).any(1))[0]
    assert bad.size == 0, f"{bad.size} superblocks differ, first {bad[:5]}"


def test_requant_full_layer_sampled(q, orc):
    """One layer of the 40-layer shape: 256 routed down matrices Q5_K
    (256 x 2048 rows of 512) and the shared expert's three Q8_0 matrices."""
    cfg = wl.CONFIGS["stack"]
    gu.banner("requant full layer: routed down Q5_K + shared Q8_0, sampled superblocks")
    W = wl.layer_weights(cfg, 0, "cuda", shared_type=wl.Q8_0, down_type=wl.Q5_K)
    rng = np.random.default_rng(5)
    cases = [("down", wl.Q5_K, cfg.E * cfg.H, cfg.F), ("sgate", wl.Q8_0, cfg.Fs, cfg.H),
             ("sup", wl.Q8_0, cfg.Fs, cfg.H), ("sdown", wl.Q8_0, cfg.H, cfg.Fs)]
    for name, st, n_rows, K in cases:
        src = W[name]
        dst = _run(q, src, st, n_rows, K)
        n_sb = n_rows * (K // 256)
        sb_bytes = wl.row_bytes(st, 256)
        pick = rng.choice(n_sb, min(n_sb, 3000), replace=False)
        s_host = gu.host(src).reshape(n_sb, sb_bytes)[pick]
        ref = orc.requant_q4k(s_host.reshape(-1), st, len(pick), 256).reshape(-1, 144)
        got = gu.host(dst).reshape(n_sb, 144)[pick]
        assert np.array_equal(got, ref), name
        print(f"  {name}: {n_sb} superblocks, {len(pick)} sampled, identical", flush=True)
