"""Pins of the oracle's Q8_1 quantiser, integer sub-block dots and row dots.

Against: hand-worked Q8_1 blocks (tests/golden/q8_1_blocks.txt), quantiser
invariants, numpy int64 dots of independently decoded codes, and the dense
reconstruction identity (the row value equals the fp64 dot of the decoded
weights with the decoded activations, up to the fp16 rounding of the stored
activation sum).
"""
import os

import numpy as np
import pytest

import qformats as qf
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _cases():
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, "q8_1_blocks.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "case":
            cur = {}
            cases.append(cur)
        else:
            cur[key] = rest
    return cases


@pytest.mark.parametrize("ci", [0, 1, 2])
def test_q8_1_handworked(orc, ci):
    c = _cases()[ci]
    x = np.zeros(32, np.float32)
    xv = [float(t) for t in c["x"].split()]
    x[:len(xv)] = xv
    blk = orc.quantize_q8_1(x)
    d = int(c["d"], 16)
    s = int(c["s"], 16)
    assert int(blk[0]) | (int(blk[1]) << 8) == d
    assert int(blk[2]) | (int(blk[3]) << 8) == s
    q = np.zeros(32, np.int64)
    qv = [int(t) for t in c["q"].split()]
    q[:len(qv)] = qv
    assert np.array_equal(blk[4:].view(np.int8).astype(np.int64), q)


def test_q8_1_invariants(orc):
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((500, 32)) * 10.0 ** rng.uniform(-4, 3, (500, 1))).astype(np.float32)
    x[::7, 5] = 0.0
    blocks = orc.quantize_q8_1(x.ravel()).reshape(500, 36)
    d, s, q = qf.q8_fields(blocks, qf.Q8_1)
    amax = np.abs(x).max(1)
    # the largest-magnitude element takes the code +-127
    i = np.abs(x).argmax(1)
    assert np.all(np.abs(q[np.arange(500), i]) == 127)
    assert np.all(np.sign(q[np.arange(500), i]) == np.sign(x[np.arange(500), i]))
    assert np.abs(q).max() <= 127
    # codes are within half a step of x / (amax/127) (fp32 scale)
    d32 = (amax / np.float32(127)).astype(np.float64)
    assert np.all(np.abs(x / d32[:, None] - q) <= 0.5 + 1e-5)
    # stored d is the fp16 of the fp32 scale; stored s represents d16 * sum(q)
    # (fp16 rounding: half an ulp, 2^-11 relative for normals, 2^-25 absolute for subnormals)
    assert np.all(np.abs(d - d32) <= np.maximum(d32 * 2.0 ** -11, 2.0 ** -25))
    exact = d * q.sum(1)
    assert np.all(np.abs(s - exact) <= np.maximum(np.abs(exact) * 2.0 ** -11, 2.0 ** -25))
    # zero block
    z = orc.quantize_q8_1(np.zeros(64, np.float32))
    assert not z.any()


def _random_xq(orc, n, seed):
    x = np.random.default_rng(seed).standard_normal(n).astype(np.float32)
    return orc.quantize_q8_1(x)


@pytest.mark.parametrize("typ,K", [(qf.Q4_K, 2048), (qf.Q5_K, 512), (qf.Q8_0, 2048), (qf.Q4_K, 256), (qf.Q5_K, 768)])
def test_subblock_dots_integer_exact(orc, typ, K):
    rows = wl.quantize(wl.randn((8, K), 21 + K) * 0.02, typ).numpy()
    xq = _random_xq(orc, K, 22 + typ)
    _, _, qa = qf.q8_fields(xq, qf.Q8_1)
    qa = qa.reshape(-1)
    for r in range(8):
        got = orc.subblock_dots(rows[r], typ, K, xq)
        qw = qf.codes(rows[r], typ)
        want = (qw.reshape(-1, 32) * qa.reshape(-1, 32)).sum(1)
        assert np.array_equal(got, want)


@pytest.mark.parametrize("typ,K", [(qf.Q4_K, 2048), (qf.Q5_K, 512), (qf.Q8_0, 2048), (qf.Q4_K, 768)])
def test_row_dot_dense_reconstruction(orc, typ, K):
    """row value == sum_i deq(w_i) * deq(a_i) up to the fp16 rounding of the
    stored activation sums (only the K-quant min term reads them)."""
    rows = wl.quantize(wl.randn((16, K), 31 + K) * 0.02, typ).numpy()
    xq = _random_xq(orc, K, 32 + typ)
    da, sa, qa = qf.q8_fields(xq, qf.Q8_1)
    a = (da[:, None] * qa).reshape(-1)
    for r in range(16):
        w = qf.decode(rows[r], typ)
        dense = float(np.dot(w, a))
        got = orc.row_dot(rows[r], typ, K, xq)
        if typ == qf.Q8_0:
            bound = 0.0
        else:
            _, dmin, _, m = qf.kquant_fields(rows[r].reshape(-1, qf.NB[typ]))
            mins = (dmin[:, None] * m).reshape(-1)                  # per 32-element sub-block
            bound = float(np.sum(mins * np.abs(sa - da * qa.sum(1))))
        noise = 1e-12 * float(np.sum(np.abs(w * a))) + 1e-300
        assert abs(got - dense) <= bound + noise, (r, got, dense, bound)


def test_row_dot_min_term_uses_stored_sum(orc):
    """A block whose codes are all zero isolates the min term: the row value is
    -sum_j dmin*m_j*s_j exactly, read from the stored activation sums."""
    K = 256
    d = np.float16(0.5)
    dmin = np.float16(0.25)
    sc = np.arange(1, 9)
    m = np.array([3, 1, 4, 1, 5, 9, 2, 6])
    import torch
    blk = wl.assemble_kquant(torch.tensor([float(d)]), torch.tensor([float(dmin)]),
                             torch.from_numpy(sc[None]), torch.from_numpy(m[None]),
                             torch.zeros(1, 256, dtype=torch.int64), wl.Q4_K).numpy().ravel()
    xq = _random_xq(orc, K, 41)
    _, sa, _ = qf.q8_fields(xq, qf.Q8_1)
    want = -float(np.sum(0.25 * m * sa))
    assert orc.row_dot(blk, qf.Q4_K, K, xq) == want
