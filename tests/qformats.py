"""Test-side numpy decoders of the weight/activation block formats.

Written separately from the oracle's C decoders (vectorised numpy, fields
taken straight from the GGUF layout reading) so the two can pin each other;
the hand-worked golden blocks pin both to the layout itself.
"""
import numpy as np

Q8_0, Q8_1, Q4_K, Q5_K = 8, 9, 12, 13
NB = {Q4_K: 144, Q5_K: 176, Q8_0: 34, Q8_1: 36}


def f16(lo, hi):
    return (lo.astype(np.uint16) | (hi.astype(np.uint16) << 8)).view(np.float16).astype(np.float64)


def kquant_fields(blocks):
    """blocks uint8 [n, 144 or 176] -> d, dmin [n]; sc, m [n, 8] (int)."""
    b = blocks
    d = f16(b[:, 0], b[:, 1])
    dmin = f16(b[:, 2], b[:, 3])
    s = b[:, 4:16].astype(np.int64)
    sc = np.empty((b.shape[0], 8), np.int64)
    m = np.empty((b.shape[0], 8), np.int64)
    sc[:, :4] = s[:, 0:4] & 0x3F
    m[:, :4] = s[:, 4:8] & 0x3F
    sc[:, 4:] = (s[:, 8:12] & 0x0F) | ((s[:, 0:4] >> 6) << 4)
    m[:, 4:] = (s[:, 8:12] >> 4) | ((s[:, 4:8] >> 6) << 4)
    return d, dmin, sc, m


def kquant_codes(blocks, typ):
    """-> int codes [n, 256]."""
    n = blocks.shape[0]
    qs_off = 16 if typ == Q4_K else 48
    qs = blocks[:, qs_off:qs_off + 128].astype(np.int64).reshape(n, 4, 32)
    q = np.empty((n, 4, 2, 32), np.int64)
    q[:, :, 0, :] = qs & 0x0F
    q[:, :, 1, :] = qs >> 4
    if typ == Q5_K:
        qh = blocks[:, 16:48].astype(np.int64)            # [n, 32]
        for g in range(4):
            q[:, g, 0, :] |= ((qh >> (2 * g)) & 1) << 4
            q[:, g, 1, :] |= ((qh >> (2 * g + 1)) & 1) << 4
    return q.reshape(n, 256)


def decode_kquant(blocks, typ):
    blocks = np.asarray(blocks, np.uint8).reshape(-1, NB[typ])
    d, dmin, sc, m = kquant_fields(blocks)
    q = kquant_codes(blocks, typ).reshape(-1, 8, 32)
    w = d[:, None, None] * sc[:, :, None] * q - (dmin[:, None] * m)[:, :, None]
    return w.reshape(-1)


def q8_fields(blocks, typ):
    """Q8_0 / Q8_1 -> d [n], s [n] (Q8_1 only, else None), q int [n, 32]."""
    blocks = np.asarray(blocks, np.uint8).reshape(-1, NB[typ])
    d = f16(blocks[:, 0], blocks[:, 1])
    if typ == Q8_1:
        s = f16(blocks[:, 2], blocks[:, 3])
        q = blocks[:, 4:36].view(np.int8).astype(np.int64)
    else:
        s = None
        q = blocks[:, 2:34].view(np.int8).astype(np.int64)
    return d, s, q


def decode(blocks, typ):
    if typ in (Q4_K, Q5_K):
        return decode_kquant(blocks, typ)
    d, _, q = q8_fields(blocks, typ)
    return (d[:, None] * q).reshape(-1)


def codes(blocks, typ):
    """Integer codes of every element of a row of blocks (flat)."""
    if typ in (Q4_K, Q5_K):
        return kquant_codes(np.asarray(blocks, np.uint8).reshape(-1, NB[typ]), typ).reshape(-1)
    return q8_fields(blocks, typ)[2].reshape(-1)


def matrix(blob, typ, rows, K):
    """Decode a [rows][K] matrix of blocks into fp64 [rows, K]."""
    return decode(np.asarray(blob, np.uint8).reshape(-1), typ).reshape(rows, K)
