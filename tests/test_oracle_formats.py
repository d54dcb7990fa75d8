"""Pins of the oracle's scalar conversions and block decoders.

Against: numpy/torch conversions (library routines), the hand-worked golden
blocks in tests/golden/, and an independently written numpy decoder.
"""
import os

import numpy as np
import pytest
import torch

import qformats as qf
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------ conversions
def _f16_cases():
    rng = np.random.default_rng(1)
    vals = [0.0, -0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 1e6, -1e6, np.inf, -np.inf,
            2.0 ** -14, 2.0 ** -24, 2.0 ** -25, 2.0 ** -25 * 1.0000001, 3 * 2.0 ** -25, 2.0 ** -26,
            1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11, 1e-8, 6.1e-5, 5.96e-8]
    vals += list(rng.standard_normal(4000) * 10.0 ** rng.uniform(-9, 5, 4000))
    # exact halfway points between adjacent binary16 values (normal and subnormal)
    h = np.arange(0, 0x7BFF, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    h2 = np.arange(1, 0x7C00, 37, dtype=np.uint16).view(np.float16).astype(np.float64)
    n = min(h.size, h2.size)
    vals += list(((h[:n] + h2[:n]) / 2))
    return np.array(vals, dtype=np.float32)


def test_f32_to_f16_matches_numpy(orc):
    x = _f16_cases()
    x = np.concatenate([x, -x])
    got = orc.f32_to_f16(x)
    want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want)


def test_f32_to_bf16_matches_torch(orc):
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(5000) * 10.0 ** rng.uniform(-30, 30, 5000)).astype(np.float32)
    # exact ties: low 16 bits 0x8000 with even and odd kept parts
    u = rng.integers(0, 2 ** 31 - 2 ** 24, 2000, dtype=np.int64).astype(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).astype(np.uint32).view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38, 1e-40, 3.3895314e38], np.float32)
    x = np.concatenate([x, ties, special])
    got = orc.f32_to_bf16(x)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want)


def test_f16_and_bf16_decode_all_patterns(orc):
    pats = np.arange(0, 65536, 1, dtype=np.uint32).astype(np.uint16)
    f16 = pats.view(np.float16).astype(np.float64)
    got = orc.f16_to_f64(pats)
    ok = np.isnan(f16)
    assert np.array_equal(got[~ok], f16[~ok]) and np.all(np.isnan(got[ok]))
    bf = (pats.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    got = orc.bf16_to_f64(pats)
    ok = np.isnan(bf)
    assert np.array_equal(got[~ok], bf[~ok]) and np.all(np.isnan(got[ok]))


# ------------------------------------------------------------ golden blocks
def _read_golden(name):
    blocks, cur = [], None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key in ("block", "case"):
            cur = {"name": rest, "expect": []}
            blocks.append(cur)
        elif key == "expect":
            i, v = rest.split()
            cur["expect"].append((int(i), float(v)))
        else:
            cur[key] = rest
    return blocks


def _hex16(s):
    v = int(s, 16)
    return [v & 0xFF, v >> 8]


def _build_kquant(g, typ):
    qs = np.zeros(128, np.uint8)
    for n in range(128):
        if g["qs_rule"] == "n%16*0x11":
            qs[n] = (n % 16) * 0x11
        elif g["qs_rule"] == "n%16|(n//8%16)<<4":
            qs[n] = (n % 16) | (((n // 8) % 16) << 4)
        else:
            raise ValueError(g["qs_rule"])
    head = _hex16(g["d"]) + _hex16(g["dmin"]) + [int(t, 16) for t in g["scales"].split()]
    if typ == qf.Q5_K:
        assert g["qh_rule"] == "0x0F if l<16 else 0xF0"
        qh = [0x0F if l < 16 else 0xF0 for l in range(32)]
        blk = np.array(head + qh + list(qs), np.uint8)
    else:
        blk = np.array(head + list(qs), np.uint8)
    assert blk.size == (144 if typ == qf.Q4_K else 176)
    return blk


@pytest.mark.parametrize("which", ["A", "B"])
def test_q4k_handworked(orc, which):
    g = [b for b in _read_golden("q4k_blocks.txt") if b["name"] == which][0]
    blk = _build_kquant(g, qf.Q4_K)
    got = orc.decode(blk, orc.Q4_K)
    for i, v in g["expect"]:
        assert got[i] == v, (which, i, got[i], v)
    if "sc" in g:
        sc, m = orc.kquant_scales(blk)
        assert list(sc) == [int(t) for t in g["sc"].split()]
        assert list(m) == [int(t) for t in g["m"].split()]
    # the independent numpy decoder agrees on the whole block
    assert np.array_equal(got, qf.decode(blk, qf.Q4_K))


def test_q5k_handworked(orc):
    g = _read_golden("q5k_block.txt")[0]
    blk = _build_kquant(g, qf.Q5_K)
    got = orc.decode(blk, orc.Q5_K)
    for i, v in g["expect"]:
        assert got[i] == v, (i, got[i], v)
    assert np.array_equal(got, qf.decode(blk, qf.Q5_K))


def test_q8_0_handworked(orc):
    g = _read_golden("q8_0_block.txt")[0]
    q = np.array([i - 16 for i in range(32)], np.int8).view(np.uint8)
    blk = np.array(_hex16(g["d"]) + list(q), np.uint8)
    assert blk.size == 34
    got = orc.decode(blk, orc.Q8_0)
    for i, v in g["expect"]:
        assert got[i] == v
    assert np.array_equal(got, qf.decode(blk, qf.Q8_0))


# ------------------------------------------------------------ packing round trips
def test_scale_packing_all_values(orc):
    """Every (sc, m) pair in 0..63 x 0..63 at each of the 8 sub-block positions
    survives the generator's packer and the oracle's / numpy's unpackers."""
    vals = np.arange(64)
    sc_all, m_all = np.meshgrid(vals, vals, indexing="ij")
    sc_all, m_all = sc_all.ravel(), m_all.ravel()            # 4096 pairs
    rng = np.random.default_rng(3)
    for pos in range(8):
        sc = rng.integers(0, 64, (4096, 8))
        m = rng.integers(0, 64, (4096, 8))
        sc[:, pos] = sc_all
        m[:, pos] = m_all
        q = rng.integers(0, 16, (4096, 256))
        d = torch.full((4096,), 0.5)
        blocks = wl.assemble_kquant(d, d, torch.from_numpy(sc), torch.from_numpy(m), torch.from_numpy(q), wl.Q4_K).numpy()
        _, _, sc2, m2 = qf.kquant_fields(blocks)
        assert np.array_equal(sc2, sc) and np.array_equal(m2, m)
        for r in range(0, 4096, 257):
            s3, m3 = orc.kquant_scales(blocks[r])
            assert np.array_equal(s3, sc[r]) and np.array_equal(m3, m[r])
        assert np.array_equal(qf.kquant_codes(blocks, qf.Q4_K), q)


@pytest.mark.parametrize("typ", [qf.Q4_K, qf.Q5_K, qf.Q8_0])
def test_random_blocks_oracle_vs_numpy(orc, typ):
    rng = np.random.default_rng(4 + typ)
    nb = qf.NB[typ]
    blocks = rng.integers(0, 256, (300, nb)).astype(np.uint8)
    # keep d/dmin finite: clear the top exponent bit of the f16 fields
    blocks[:, 1] &= 0x3F
    if typ != qf.Q8_0:
        blocks[:, 3] &= 0x3F
    got = orc.decode(blocks.ravel(), typ)
    want = qf.decode(blocks, typ)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("typ", [qf.Q4_K, qf.Q5_K])
def test_codes_roundtrip_through_generator(orc, typ):
    rng = np.random.default_rng(7)
    nmax = 15 if typ == qf.Q4_K else 31
    q = rng.integers(0, nmax + 1, (64, 256))
    sc = rng.integers(0, 64, (64, 8))
    m = rng.integers(0, 64, (64, 8))
    d = torch.from_numpy(rng.uniform(0.001, 0.01, 64).astype(np.float32))
    dm = torch.from_numpy(rng.uniform(0.001, 0.01, 64).astype(np.float32))
    blocks = wl.assemble_kquant(d, dm, torch.from_numpy(sc), torch.from_numpy(m), torch.from_numpy(q), typ).numpy()
    assert np.array_equal(qf.kquant_codes(blocks, typ), q)
    dd = d.to(torch.float16).double().numpy()
    dmd = dm.to(torch.float16).double().numpy()
    want = (dd[:, None, None] * sc[:, :, None] * q.reshape(64, 8, 32) - (dmd[:, None] * m)[:, :, None]).reshape(-1)
    assert np.array_equal(orc.decode(blocks.ravel(), typ), want)


@pytest.mark.parametrize("typ", [qf.Q4_K, qf.Q5_K, qf.Q8_0])
def test_generator_quantiser_error_bound(orc, typ):
    """The generator's weight encoder reproduces N(0, 0.02) draws to within its
    step size (data sanity: the bytes the workloads use are well formed)."""
    x = wl.randn((16, 512), 11) * 0.02
    blob = wl.quantize(x, typ).numpy()
    deq = orc.decode(blob.ravel(), typ).reshape(16, 512)
    err = np.abs(deq - x.double().numpy())
    assert err.max() < 0.02 * (0.35 if typ == qf.Q4_K else 0.2)
