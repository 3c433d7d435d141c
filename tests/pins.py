"""Pins for the CPU oracle: checks tied to something other than the oracle
itself (hand-assembled blocks with hand-computed values, exact rational
arithmetic, numpy's binary16 conversion, brute-force sums, closed forms).

Each ``pin_*`` takes an oracle object and raises AssertionError on a
mismatch, so the same pins run against the real oracle and against mutants
built from edited copies of its source (which must fail at least one pin).

The test-side encoders below write blocks from field values; they are a
second, independent statement of each layout (the oracle only decodes).
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K = 5, 6, 7, 8, 9
BLOCK = {Q4_K: (256, 144), Q6_K: (256, 210), Q4_0: (32, 18), Q8_0: (32, 36), Q8_0_F16: (32, 34), Q5_1: (32, 24),
         Q5_K: (256, 176), Q2_K: (256, 84), Q3_K: (256, 110)}


def golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def block_of(g: dict) -> np.ndarray:
    return np.frombuffer(bytes.fromhex(g["block_hex"]), dtype=np.uint8).copy()


# ---------------------------------------------------------------- encoders

def f16_bits(v) -> np.ndarray:
    return np.asarray(v, dtype=np.float16).view(np.uint16)


def encode_q4_K(d16, dmin16, sc, mn, q) -> bytes:
    """Q4_K blocks from fields (batched over a leading axis): d/dmin as fp16
    bit patterns [nb], sc/mn six-bit values [nb, 8], q nibbles [nb, 256] in
    weight order."""
    d16 = np.atleast_1d(np.asarray(d16, dtype=np.uint16))
    dmin16 = np.atleast_1d(np.asarray(dmin16, dtype=np.uint16))
    sc = np.asarray(sc, dtype=np.int64).reshape(len(d16), 8)
    mn = np.asarray(mn, dtype=np.int64).reshape(len(d16), 8)
    q = np.asarray(q, dtype=np.int64).reshape(len(d16), 256)
    out = np.zeros((len(d16), 144), dtype=np.uint8)
    out[:, 0:2] = d16.view(np.uint8).reshape(-1, 2)
    out[:, 2:4] = dmin16.view(np.uint8).reshape(-1, 2)
    for j in range(4):
        out[:, 4 + j] = (sc[:, j] & 63) | ((sc[:, j + 4] >> 4) << 6)
        out[:, 8 + j] = (mn[:, j] & 63) | ((mn[:, j + 4] >> 4) << 6)
        out[:, 12 + j] = (sc[:, j + 4] & 15) | ((mn[:, j + 4] & 15) << 4)
    for g in range(4):
        out[:, 16 + 32 * g:16 + 32 * g + 32] = q[:, 64 * g:64 * g + 32] | (q[:, 64 * g + 32:64 * g + 64] << 4)
    return out.tobytes()


def encode_q6_K(d16, scales, q) -> bytes:
    """Q6_K blocks from fields (batched): d as fp16 bits [nb], int8 scales
    [nb, 16], signed codes in [-32, 31] [nb, 256] in weight order."""
    d16 = np.atleast_1d(np.asarray(d16, dtype=np.uint16))
    nb = len(d16)
    u = np.asarray(q, dtype=np.int64).reshape(nb, 256) + 32
    out = np.zeros((nb, 210), dtype=np.int64)
    for i in range(256):
        h, k, l = i // 128, (i % 128) // 32, i % 32
        lo, hi = u[:, i] & 15, u[:, i] >> 4
        idx = 64 * h + 32 * (k & 1) + l
        out[:, idx] |= lo if k < 2 else (lo << 4)
        out[:, 128 + 32 * h + l] |= hi << (2 * k)
    out[:, 192:208] = np.asarray(scales, dtype=np.int64).reshape(nb, 16) & 0xFF
    res = out.astype(np.uint8)
    res[:, 208:210] = d16.view(np.uint8).reshape(-1, 2)
    return res.tobytes()


def encode_q8_0(scale32, q) -> bytes:
    s = np.atleast_1d(np.asarray(scale32, dtype=np.float32))
    out = np.zeros((len(s), 36), dtype=np.uint8)
    out[:, 0:4] = s.view(np.uint8).reshape(-1, 4)
    out[:, 4:] = (np.asarray(q, dtype=np.int64).reshape(len(s), 32) & 0xFF).astype(np.uint8)
    return out.tobytes()


def encode_q4_0(d16, nib) -> bytes:
    d16 = np.atleast_1d(np.asarray(d16, dtype=np.uint16))
    nib = np.asarray(nib, dtype=np.int64).reshape(len(d16), 32)
    out = np.zeros((len(d16), 18), dtype=np.uint8)
    out[:, 0:2] = d16.view(np.uint8).reshape(-1, 2)
    out[:, 2:] = nib[:, :16] | (nib[:, 16:] << 4)
    return out.tobytes()


# The ggml-layout formats (a reading of the pages, which give only Q2_K's
# size): each encoder writes the fields at the offsets the format fixes.

def encode_q8_0_f16(d16, q) -> bytes:
    d16 = np.atleast_1d(np.asarray(d16, dtype=np.uint16))
    out = np.zeros((len(d16), 34), dtype=np.uint8)
    out[:, 0:2] = d16.view(np.uint8).reshape(-1, 2)
    out[:, 2:] = (np.asarray(q, dtype=np.int64).reshape(len(d16), 32) & 0xFF).astype(np.uint8)
    return out.tobytes()


def encode_q5_1(d16, m16, q) -> bytes:
    """q: five-bit codes [nb, 32] in weight order."""
    d16 = np.atleast_1d(np.asarray(d16, dtype=np.uint16))
    m16 = np.atleast_1d(np.asarray(m16, dtype=np.uint16))
    nb = len(d16)
    q = np.asarray(q, dtype=np.int64).reshape(nb, 32)
    out = np.zeros((nb, 24), dtype=np.uint8)
    out[:, 0:2] = d16.view(np.uint8).reshape(-1, 2)
    out[:, 2:4] = m16.view(np.uint8).reshape(-1, 2)
    qh = np.zeros(nb, dtype=np.uint64)
    for i in range(32):
        qh |= ((q[:, i] >> 4) & 1).astype(np.uint64) << np.uint64(i)
    out[:, 4:8] = qh.astype(np.uint32).view(np.uint8).reshape(-1, 4)
    out[:, 8:] = (q[:, :16] & 15) | ((q[:, 16:] & 15) << 4)
    return out.tobytes()


def _pack_k4_scales(sc, mn) -> np.ndarray:
    out = np.zeros((len(sc), 12), dtype=np.int64)
    for j in range(4):
        out[:, j] = (sc[:, j] & 63) | ((sc[:, j + 4] >> 4) << 6)
        out[:, 4 + j] = (mn[:, j] & 63) | ((mn[:, j + 4] >> 4) << 6)
        out[:, 8 + j] = (sc[:, j + 4] & 15) | ((mn[:, j + 4] & 15) << 4)
    return out


def encode_q5_K(d16, dmin16, sc, mn, q) -> bytes:
    """q: five-bit codes [nb, 256] in weight order; sc/mn [nb, 8]."""
    d16 = np.atleast_1d(np.asarray(d16, dtype=np.uint16))
    dmin16 = np.atleast_1d(np.asarray(dmin16, dtype=np.uint16))
    nb = len(d16)
    sc = np.asarray(sc, dtype=np.int64).reshape(nb, 8)
    mn = np.asarray(mn, dtype=np.int64).reshape(nb, 8)
    q = np.asarray(q, dtype=np.int64).reshape(nb, 256)
    out = np.zeros((nb, 176), dtype=np.int64)
    out[:, 4:16] = _pack_k4_scales(sc, mn)
    for g in range(4):
        lo, hi = q[:, 64 * g:64 * g + 32], q[:, 64 * g + 32:64 * g + 64]
        out[:, 48 + 32 * g:48 + 32 * g + 32] = (lo & 15) | ((hi & 15) << 4)
        out[:, 16:48] |= ((lo >> 4) << (2 * g)) | ((hi >> 4) << (2 * g + 1))
    res = out.astype(np.uint8)
    res[:, 0:2] = d16.view(np.uint8).reshape(-1, 2)
    res[:, 2:4] = dmin16.view(np.uint8).reshape(-1, 2)
    return res.tobytes()


def encode_q2_K(d16, dmin16, sc, mn, q) -> bytes:
    """sc/mn: four-bit scale and min per 16 weights [nb, 16]; q: codes 0..3
    [nb, 256] in weight order."""
    d16 = np.atleast_1d(np.asarray(d16, dtype=np.uint16))
    dmin16 = np.atleast_1d(np.asarray(dmin16, dtype=np.uint16))
    nb = len(d16)
    q = np.asarray(q, dtype=np.int64).reshape(nb, 256)
    out = np.zeros((nb, 84), dtype=np.int64)
    out[:, 0:16] = (np.asarray(sc, dtype=np.int64).reshape(nb, 16) & 15) | \
        ((np.asarray(mn, dtype=np.int64).reshape(nb, 16) & 15) << 4)
    for i in range(256):
        h, j, l = i // 128, (i % 128) // 32, i % 32
        out[:, 16 + 32 * h + l] |= q[:, i] << (2 * j)
    res = out.astype(np.uint8)
    res[:, 80:82] = d16.view(np.uint8).reshape(-1, 2)
    res[:, 82:84] = dmin16.view(np.uint8).reshape(-1, 2)
    return res.tobytes()


def encode_q3_K(d16, scales, q) -> bytes:
    """scales: signed scale values -32..31 per 16 weights [nb, 16]; q: codes
    -4..3 [nb, 256] in weight order."""
    d16 = np.atleast_1d(np.asarray(d16, dtype=np.uint16))
    nb = len(d16)
    u = np.asarray(scales, dtype=np.int64).reshape(nb, 16) + 32
    q = np.asarray(q, dtype=np.int64).reshape(nb, 256) + 4
    out = np.zeros((nb, 110), dtype=np.int64)
    for i in range(256):
        h, j, l = i // 128, (i % 128) // 32, i % 32
        out[:, 32 + 32 * h + l] |= (q[:, i] & 3) << (2 * j)
        out[:, l] |= (q[:, i] >> 2) << (4 * h + j)
    for s in range(16):
        lo, hi = u[:, s] & 15, u[:, s] >> 4
        out[:, 96 + (s % 8)] |= lo << (0 if s < 8 else 4)
        out[:, 96 + 8 + s % 4] |= hi << (2 * (s // 4))
    res = out.astype(np.uint8)
    res[:, 108:110] = d16.view(np.uint8).reshape(-1, 2)
    return res.tobytes()


# ---------------------------------------------------------------- pins

def pin_block_sizes(o):
    """Bytes per block match the pages' bits per weight: Q4_K 4.50 and Q6_K
    6.56 ("picoLM, in Python", §2 K-quants), q4_0 4.5 (PETIT, "What makes it
    fast & small"); q8_0 is a 4-byte scale plus 32 int8 (PETIT, "How the
    pieces match")."""
    assert o.block_elems(Q4_K) == 256 and o.block_bytes(Q4_K) == 144
    assert o.block_elems(Q6_K) == 256 and o.block_bytes(Q6_K) == 210
    assert o.block_elems(Q4_0) == 32 and o.block_bytes(Q4_0) == 18
    assert o.block_elems(Q8_0) == 32 and o.block_bytes(Q8_0) == 36
    assert 8 * 144 / 256 == 4.5
    assert round(8 * 210 / 256, 2) == 6.56
    assert 8 * 18 / 32 == 4.5
    assert o.block_elems(99) < 0 and o.block_bytes(0) < 0


def pin_ggml_block_sizes(o):
    """Q2_K: 84 bytes per 256 weights, 2.62 bits/weight ("picoLM, in
    Python", §2, the bits-per-weight lines). The other ggml-layout sizes
    follow from their fields: Q3_K 32+64+12+2, Q5_K 2+2+12+32+128, Q5_1
    2+2+4+16, GGUF Q8_0 2+32."""
    assert o.block_elems(Q2_K) == 256 and o.block_bytes(Q2_K) == 84
    assert abs(8 * 84 / 256 - 2.62) < 0.01
    for t, (qk, bb) in BLOCK.items():
        assert o.block_elems(t) == qk and o.block_bytes(t) == bb, t


def pin_half_to_float(o):
    """binary16 -> binary32 agrees with numpy's conversion on all 65536
    patterns (NaN compared as a class)."""
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float32)
    got = np.array([o.half_to_float(int(b)) for b in bits], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def pin_bf16(o):
    for b in (0x0000, 0x8000, 0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F, 0xFF7F, 0x7F80):
        ref = np.array([b << 16], dtype=np.uint32).view(np.float32)[0]
        assert np.float32(o.bf16_to_float(b)).view(np.uint32) == ref.view(np.uint32)


def pin_q4k_h1(o):
    g = golden("q4k_h1.json")
    w = o.dequantize_row(Q4_K, block_of(g), 256)
    for i, v in g["expected"].items():
        assert w[int(i)] == v, (i, w[int(i)], v)
    assert float(np.sum(w.astype(np.float64))) == g["sum"]
    # hand rule for every weight (d = 1, dmin = 0.5)
    sc, mn = g["fields"]["sc"], g["fields"]["mn"]
    for gi in range(4):
        for l in range(32):
            assert w[64 * gi + l] == sc[2 * gi] * (l & 15) - 0.5 * mn[2 * gi]
            assert w[64 * gi + 32 + l] == sc[2 * gi + 1] * (15 - (l & 15)) - 0.5 * mn[2 * gi + 1]


def pin_q6k_h2(o):
    g = golden("q6k_h2.json")
    w = o.dequantize_row(Q6_K, block_of(g), 256)
    for i, v in g["expected"].items():
        assert w[int(i)] == v, (i, w[int(i)], v)
    sc = g["fields"]["scales"]
    assert all(w[i] == sc[i // 16] for i in range(256))


def pin_q6k_h3(o):
    g = golden("q6k_h3.json")
    w = o.dequantize_row(Q6_K, block_of(g), 256)
    for i in range(256):
        want = g["expected"].get(str(i), g["default"])
        assert w[i] == want, (i, w[i], want)


def pin_q8_0_hand(o):
    g = golden("q8_0_hand.json")
    w = o.dequantize_row(Q8_0, block_of(g), 32)
    assert w.tolist() == g["expected_all"]


def pin_q4_0_hand(o):
    g = golden("q4_0_hand.json")
    w = o.dequantize_row(Q4_0, block_of(g), 32)
    assert w.tolist() == g["expected_all"]


def pin_q8_0_f16_hand(o):
    g = golden("q8_0_f16_hand.json")
    w = o.dequantize_row(Q8_0_F16, block_of(g), 32)
    assert w.tolist() == g["expected_all"]


def pin_q5_1_hand(o):
    g = golden("q5_1_hand.json")
    w = o.dequantize_row(Q5_1, block_of(g), 32)
    assert w.tolist() == g["expected_all"]


def pin_q5k_hand(o):
    g = golden("q5k_hand.json")
    w = o.dequantize_row(Q5_K, block_of(g), 256)
    for i, v in g["expected"].items():
        assert w[int(i)] == v, (i, w[int(i)], v)
    f = g["fields"]
    sc, mn = f["sc"], f["mn"]
    for gi in range(4):
        for l in range(32):
            qh = f["qh_lo"] if l < 16 else f["qh_hi"]
            lo = (l & 15) + 16 * ((qh >> (2 * gi)) & 1)
            hi = 15 - (l & 15) + 16 * ((qh >> (2 * gi + 1)) & 1)
            assert w[64 * gi + l] == sc[2 * gi] * lo - 0.5 * mn[2 * gi]
            assert w[64 * gi + 32 + l] == sc[2 * gi + 1] * hi - 0.5 * mn[2 * gi + 1]


def pin_q2k_hand(o):
    g = golden("q2k_hand.json")
    w = o.dequantize_row(Q2_K, block_of(g), 256)
    for i, v in g["expected"].items():
        assert w[int(i)] == v, (i, w[int(i)], v)
    for i in range(256):
        j = (i % 128) // 32
        q = j if i < 128 else 3 - j
        assert w[i] == (i // 16) * q - (15 - i // 16), i


def pin_q3k_hand(o):
    g = golden("q3k_hand.json")
    w = o.dequantize_row(Q3_K, block_of(g), 256)
    for i, v in g["expected"].items():
        assert w[int(i)] == v, (i, w[int(i)], v)
    f = g["fields"]
    for i in range(256):
        h, j, l = i // 128, (i % 128) // 32, i % 32
        q2 = j if h == 0 else 3 - j
        hm = f["hm_lo"] if l < 16 else f["hm_hi"]
        q = q2 - (0 if (hm >> (4 * h + j)) & 1 else 4)
        assert w[i] == f["scales"][i // 16] * q, i


def _exact_check(o, t, blocks: bytes, exact64: np.ndarray, n: int):
    """Decoded weights must equal the exact value rounded once to fp32."""
    w = o.dequantize_row(t, np.frombuffer(blocks, dtype=np.uint8), n)
    ref = exact64.astype(np.float32)
    assert np.array_equal(w.view(np.uint32), ref.view(np.uint32)), np.flatnonzero(w != ref)[:8]


def _fp16_scales(rng, n, extremes=True):
    """fp16 scale patterns: random normals plus subnormal / tiny / huge ones."""
    v = f16_bits(rng.uniform(1e-4, 4.0, n))
    if extremes:
        v[:8] = [0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x0000, 0x1400, 0x5BFF]
    return v


def pin_q4k_exact(o, nblocks=3000, seed=11):
    """Random Q4_K fields, written by the test encoder: every decoded weight
    equals RN_fp32(d*sc*q - dmin*mn) taken exactly (the products have at most
    21 significant bits and the difference spans at most 50 bits, so float64
    holds it exactly; a sample is re-checked with Fractions)."""
    rng = np.random.default_rng(seed)
    d = _fp16_scales(rng, nblocks)
    dm = _fp16_scales(rng, nblocks)[::-1].copy()
    sc = rng.integers(0, 64, (nblocks, 8))
    mn = rng.integers(0, 64, (nblocks, 8))
    q = rng.integers(0, 16, (nblocks, 256))
    raw = encode_q4_K(d, dm, sc, mn, q)
    d64 = d.view(np.float16).astype(np.float64)[:, None]
    dm64 = dm.view(np.float16).astype(np.float64)[:, None]
    j = np.arange(256) // 32
    exact = d64 * sc[:, j] * q - dm64 * mn[:, j]
    for b, i in [(0, 0), (1, 200), (5, 77), (7, 255), (123, 131)]:
        fr = (Fraction(float(d64[b, 0])) * int(sc[b, i // 32]) * int(q[b, i])
              - Fraction(float(dm64[b, 0])) * int(mn[b, i // 32]))
        assert fr == Fraction(float(exact[b, i]))
    _exact_check(o, Q4_K, raw, exact.reshape(-1), nblocks * 256)


def pin_q4k_exhaustive(o):
    """Every (scale, min, nibble) triple in every sub-block slot, for d/dmin
    including subnormal and the largest finite fp16: decoded weights equal
    the exact value rounded once to fp32."""
    s, m = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    s, m = s.reshape(-1), m.reshape(-1)
    j = np.arange(8)
    scj = (s[:, None] + 7 * j[None, :]) % 64
    mnj = (m[:, None] + 13 * j[None, :]) % 64
    q = (np.arange(256)[None, :] * 5 + s[:, None]) % 16
    for d16, dm16 in [(0x3C00, 0x3800), (0x0001, 0x7BFF), (0x7BFF, 0x0001), (0x2E66, 0x03FF)]:
        nb = len(s)
        raw = encode_q4_K(np.full(nb, d16), np.full(nb, dm16), scj, mnj, q)
        d64 = float(np.uint16(d16).view(np.float16))
        dm64 = float(np.uint16(dm16).view(np.float16))
        sub = np.arange(256) // 32
        exact = d64 * scj[:, sub] * q - dm64 * mnj[:, sub]
        _exact_check(o, Q4_K, raw, exact.reshape(-1), nb * 256)


def pin_q6k_exact(o, nblocks=3000, seed=12):
    """Random Q6_K fields via the test encoder: weight = d*scale*q exactly
    (at most 23 significant bits, so the fp32 result is exact)."""
    rng = np.random.default_rng(seed)
    d = _fp16_scales(rng, nblocks)
    sc = rng.integers(-128, 128, (nblocks, 16))
    q = rng.integers(-32, 32, (nblocks, 256))
    raw = encode_q6_K(d, sc, q)
    d64 = d.view(np.float16).astype(np.float64)[:, None]
    exact = d64 * sc[:, np.arange(256) // 16] * q
    assert np.array_equal(exact, exact.astype(np.float32).astype(np.float64))
    _exact_check(o, Q6_K, raw, exact.reshape(-1), nblocks * 256)


def pin_q8_0_exact(o, nblocks=2000, seed=13):
    rng = np.random.default_rng(seed)
    s = rng.uniform(1e-3, 2e-2, nblocks).astype(np.float32)
    s[:3] = [np.float32(1e-38), np.float32(1.0e36), np.float32(-0.5)]
    q = rng.integers(-128, 128, (nblocks, 32))
    raw = encode_q8_0(s, q)
    exact = s.astype(np.float64)[:, None] * q  # 24 x 8 bits: exact in float64
    _exact_check(o, Q8_0, raw, exact.reshape(-1), nblocks * 32)


def pin_q4_0_exact(o, nblocks=2000, seed=14):
    rng = np.random.default_rng(seed)
    d = _fp16_scales(rng, nblocks)
    nib = rng.integers(0, 16, (nblocks, 32))
    raw = encode_q4_0(d, nib)
    exact = d.view(np.float16).astype(np.float64)[:, None] * (nib - 8)
    _exact_check(o, Q4_0, raw, exact.reshape(-1), nblocks * 32)


def pin_q8_0_f16_exact(o, nblocks=2000, seed=21):
    rng = np.random.default_rng(seed)
    d = _fp16_scales(rng, nblocks)
    q = rng.integers(-128, 128, (nblocks, 32))
    exact = d.view(np.float16).astype(np.float64)[:, None] * q  # 11 x 8 bits: exact
    _exact_check(o, Q8_0_F16, encode_q8_0_f16(d, q), exact.reshape(-1), nblocks * 32)


def pin_q5_1_exact(o, nblocks=2000, seed=22):
    """weight = RN_fp32(q*d + m), one rounding: q*d and m are multiples of
    2^-24 below 2^21 in magnitude, so float64 holds q*d + m exactly (a
    sample is re-checked with Fractions) and rounding it once to fp32 gives
    the weight."""
    rng = np.random.default_rng(seed)
    d = _fp16_scales(rng, nblocks)
    m = f16_bits(rng.uniform(-4.0, 4.0, nblocks))
    m[:4] = [0x8001, 0xFBFF, 0x0000, 0x3C00]
    q = rng.integers(0, 32, (nblocks, 32))
    exact = d.view(np.float16).astype(np.float64)[:, None] * q + m.view(np.float16).astype(np.float64)[:, None]
    for b, i in [(0, 0), (1, 31), (2, 5), (3, 17), (9, 30)]:
        fr = Fraction(float(np.float16(d.view(np.float16)[b]))) * int(q[b, i]) + \
            Fraction(float(np.float16(m.view(np.float16)[b])))
        assert fr == Fraction(float(exact[b, i]))
    _exact_check(o, Q5_1, encode_q5_1(d, m, q), exact.reshape(-1), nblocks * 32)


def pin_q5k_exact(o, nblocks=3000, seed=23):
    """As Q4_K: d*sc*q has at most 22 significant bits, dmin*mn 17, so
    float64 holds d*sc*q - dmin*mn exactly and rounding it once gives the
    weight."""
    rng = np.random.default_rng(seed)
    d = _fp16_scales(rng, nblocks)
    dm = _fp16_scales(rng, nblocks)[::-1].copy()
    sc = rng.integers(0, 64, (nblocks, 8))
    mn = rng.integers(0, 64, (nblocks, 8))
    q = rng.integers(0, 32, (nblocks, 256))
    d64 = d.view(np.float16).astype(np.float64)[:, None]
    dm64 = dm.view(np.float16).astype(np.float64)[:, None]
    j = np.arange(256) // 32
    exact = d64 * sc[:, j] * q - dm64 * mn[:, j]
    _exact_check(o, Q5_K, encode_q5_K(d, dm, sc, mn, q), exact.reshape(-1), nblocks * 256)


def pin_q2k_exact(o, nblocks=3000, seed=24):
    rng = np.random.default_rng(seed)
    d = _fp16_scales(rng, nblocks)
    dm = _fp16_scales(rng, nblocks)[::-1].copy()
    sc = rng.integers(0, 16, (nblocks, 16))
    mn = rng.integers(0, 16, (nblocks, 16))
    q = rng.integers(0, 4, (nblocks, 256))
    d64 = d.view(np.float16).astype(np.float64)[:, None]
    dm64 = dm.view(np.float16).astype(np.float64)[:, None]
    s = np.arange(256) // 16
    exact = d64 * sc[:, s] * q - dm64 * mn[:, s]
    _exact_check(o, Q2_K, encode_q2_K(d, dm, sc, mn, q), exact.reshape(-1), nblocks * 256)


def pin_q3k_exact(o, nblocks=3000, seed=25):
    """weight = d*scale*q exactly (11 + 6 + 3 significant bits)."""
    rng = np.random.default_rng(seed)
    d = _fp16_scales(rng, nblocks)
    sc = rng.integers(-32, 32, (nblocks, 16))
    q = rng.integers(-4, 4, (nblocks, 256))
    exact = d.view(np.float16).astype(np.float64)[:, None] * sc[:, np.arange(256) // 16] * q
    assert np.array_equal(exact, exact.astype(np.float32).astype(np.float64))
    _exact_check(o, Q3_K, encode_q3_K(d, sc, q), exact.reshape(-1), nblocks * 256)


def _rand_matrix(t, rows, cols, rng):
    qk, bb = BLOCK[t]
    W = rng.integers(0, 256, rows * (cols // qk) * bb, dtype=np.uint8).reshape(-1, bb)
    if t in (Q4_K, Q5_K):
        W[:, 0:4] = f16_bits(rng.uniform(1e-3, 1e-2, 2 * len(W))).view(np.uint8).reshape(-1, 4)
    elif t == Q6_K:
        W[:, 208:210] = f16_bits(rng.uniform(1e-4, 1e-3, len(W))).view(np.uint8).reshape(-1, 2)
    elif t == Q4_0:
        W[:, 0:2] = f16_bits(rng.uniform(1e-3, 2e-2, len(W))).view(np.uint8).reshape(-1, 2)
    elif t == Q8_0:
        W[:, 0:4] = rng.uniform(1e-3, 2e-2, len(W)).astype(np.float32).view(np.uint8).reshape(-1, 4)
    elif t == Q8_0_F16:
        W[:, 0:2] = f16_bits(rng.uniform(1e-3, 2e-2, len(W))).view(np.uint8).reshape(-1, 2)
    elif t == Q5_1:
        W[:, 0:4] = f16_bits(rng.uniform(-2e-2, 2e-2, 2 * len(W))).view(np.uint8).reshape(-1, 4)
    elif t == Q2_K:
        W[:, 80:84] = f16_bits(rng.uniform(1e-3, 1e-2, 2 * len(W))).view(np.uint8).reshape(-1, 4)
    elif t == Q3_K:
        W[:, 108:110] = f16_bits(rng.uniform(1e-3, 1e-2, len(W))).view(np.uint8).reshape(-1, 2)
    return W.reshape(-1)


def pin_gemv_bruteforce(o, seed=15):
    """Tiny GEMVs: the oracle's fp64 sum is within (cols-1)*2^-53*sum|w*x|
    of the exact rational sum of the fp32 weights times fp32 x, and its
    weights are exactly the dequantised row."""
    rng = np.random.default_rng(seed)
    for t, rows, cols in [(Q4_K, 3, 256), (Q4_K, 2, 512), (Q6_K, 3, 512), (Q8_0, 4, 96), (Q4_0, 4, 128),
                          (Q8_0_F16, 3, 64), (Q5_1, 3, 96), (Q5_K, 2, 256), (Q2_K, 2, 512), (Q3_K, 3, 256)]:
        W = _rand_matrix(t, rows, cols, rng)
        x = rng.standard_normal(cols).astype(np.float32)
        y, a = o.gemv(t, W, rows, cols, x)
        rb = len(W) // rows
        for r in range(rows):
            w = o.dequantize_row(t, W[r * rb:(r + 1) * rb], cols)
            terms = [Fraction(float(w[c])) * Fraction(float(x[c])) for c in range(cols)]
            exact = sum(terms, Fraction(0))
            absx = sum((abs(v) for v in terms), Fraction(0))
            bound = (cols - 1) * 2.0 ** -53 * float(absx)
            assert abs(Fraction(y[r]) - exact) <= Fraction(bound) + Fraction(1, 10 ** 300)
            assert abs(a[r] - float(absx)) <= bound + 1e-300
        # x = e_k gives column k of the dequantised matrix, bit for bit
        for k in (0, cols // 2 + 1, cols - 1):
            e = np.zeros(cols, dtype=np.float32)
            e[k] = 1.0
            yk, _ = o.gemv(t, W, rows, cols, e)
            col = [o.dequantize_row(t, W[r * rb:(r + 1) * rb], cols)[k] for r in range(rows)]
            assert yk.tolist() == [float(v) for v in col]


def pin_gemv_h1_sum(o):
    """H1 against x = 1: y = sum of the 256 hand-computed weights = 50000."""
    g = golden("q4k_h1.json")
    y, a = o.gemv(Q4_K, block_of(g), 1, 256, np.ones(256, dtype=np.float32))
    assert y[0] == 50000.0


def pin_gemm_rows(o, seed=16):
    """GEMM row m equals the GEMV with x = bf16 -> fp32 of X[m] (exact
    widening; same sums), and a unit row of X returns a column of W."""
    rng = np.random.default_rng(seed)
    for t, rows, cols, M in [(Q4_K, 3, 512, 3), (Q6_K, 2, 256, 2), (Q4_0, 2, 64, 4), (Q8_0, 3, 64, 2),
                             (Q8_0_F16, 2, 64, 2), (Q5_1, 2, 64, 3), (Q5_K, 2, 256, 2), (Q2_K, 3, 256, 2),
                             (Q3_K, 2, 512, 2)]:
        W = _rand_matrix(t, rows, cols, rng)
        Xf = rng.standard_normal((M, cols)).astype(np.float32)
        Xb = (Xf.view(np.uint32) >> 16).astype(np.uint16)
        Xb[0, :] = 0
        Xb[0, 3] = 0x3F80  # bf16 1.0
        Y, A = o.gemm(t, W, rows, cols, Xb, M)
        for m in range(M):
            xm = (Xb[m].astype(np.uint32) << 16).view(np.float32)
            y, a = o.gemv(t, W, rows, cols, xm)
            assert Y[m].tolist() == y.tolist() and A[m].tolist() == a.tolist()
        rb = len(W) // rows
        assert Y[0].tolist() == [float(o.dequantize_row(t, W[r * rb:(r + 1) * rb], cols)[3]) for r in range(rows)]


ALL_PINS = [pin_block_sizes, pin_ggml_block_sizes, pin_half_to_float, pin_bf16, pin_q4k_h1, pin_q6k_h2, pin_q6k_h3,
            pin_q8_0_hand, pin_q4_0_hand, pin_q8_0_f16_hand, pin_q5_1_hand, pin_q5k_hand, pin_q2k_hand, pin_q3k_hand,
            pin_q4k_exact, pin_q4k_exhaustive, pin_q6k_exact, pin_q8_0_exact, pin_q4_0_exact, pin_q8_0_f16_exact,
            pin_q5_1_exact, pin_q5k_exact, pin_q2k_exact, pin_q3k_exact, pin_gemv_bruteforce, pin_gemv_h1_sum,
            pin_gemm_rows]


# ---------------------------------------------------------------- the decode step and the encoder

def pin_float_to_half(o):
    """fp32 -> fp16 rounding agrees with numpy's (round to nearest even) on
    every fp16 value, every midpoint between neighbours (ties go to even),
    overflow boundaries, subnormals, infinities and NaN."""
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    vals = h.view(np.float16).astype(np.float32)
    nxt = (h + 1).view(np.float16).astype(np.float64)
    mids = ((vals.astype(np.float64) + nxt) / 2).astype(np.float32)  # exact in fp32
    rng = np.random.default_rng(31)
    rnd = (rng.standard_normal(20000) * np.exp2(rng.integers(-30, 18, 20000))).astype(np.float32)
    edge = np.array([65504, 65519.99, 65520, 65536, 1e-8, 2.0 ** -25, 2.0 ** -24 * 1.5, 2.0 ** -14, np.inf,
                     6.0e-8, 3.0e-8, 2.0 ** -26], dtype=np.float32)
    allv = np.concatenate([vals, mids, rnd, edge])
    allv = np.concatenate([allv, -allv])
    got = o.halves(allv)
    with np.errstate(over="ignore"):
        ref = allv.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:5]
    assert (o.float_to_half(float("nan")) & 0x7C00) == 0x7C00 and (o.float_to_half(float("nan")) & 0x3FF)


def pin_rmsnorm(o):
    """Hand values: x = (3, 4), w = (2, 1/2), eps = 0: mean square 12.5, so
    out = (6, 2) / sqrt(12.5) = (1.6970562748477142, 0.5656854249492381).
    eps enters inside the root: x = 1, eps = 3 gives w / 2 exactly; with w = 1
    and eps = 0 the output's mean square is 1."""
    out = o.rmsnorm(np.array([3, 4], np.float32), np.array([2, 0.5], np.float32), 0.0)
    assert out.tolist() == [np.float32(1.6970562748477142), np.float32(0.5656854249492381)]
    w = np.linspace(-2, 2, 64).astype(np.float32)
    assert np.array_equal(o.rmsnorm(np.ones(64, np.float32), w, 3.0), w / np.float32(2))
    x = np.random.default_rng(32).standard_normal(2048).astype(np.float32) * 7
    y = o.rmsnorm(x, np.ones(2048, np.float32), 0.0).astype(np.float64)
    assert abs(np.mean(y * y) - 1.0) < 1e-6
    assert np.all(o.rmsnorm(np.zeros(8, np.float32), np.ones(8, np.float32), 1e-5) == 0)


def pin_rope(o):
    """Tables: pos 0 is the identity; head_dim 2 at pos 1 rotates by 1 rad
    (cos 1 = 0.5403023058681398, sin 1 = 0.8414709848078965); head_dim 4 at
    pos 3 rotates pair 1 by 3 * 10000^-1/2 = 0.03 rad (cos 0.03 =
    0.9995500337489875, sin 0.03 = 0.029995500202495664). The rotation pairs
    x[2i] with x[2i+1] ("picoLM, in Python", RoPE layout): e_0 of a 4-wide
    head goes to (cos, sin, 0, 0), not the NeoX (cos, 0, sin, 0). Pairs keep
    their norm, and q.k after rotation depends only on the position
    difference."""
    c, s = o.rope_table(0, 64)
    assert np.all(c == 1) and np.all(s == 0)
    c, s = o.rope_table(1, 2)
    assert c[0] == np.float32(0.5403023058681398) and s[0] == np.float32(0.8414709848078965)
    c, s = o.rope_table(3, 4)
    assert c[1] == np.float32(0.9995500337489875) and s[1] == np.float32(0.029995500202495664)
    c, s = o.rope_table(1, 4)
    out = o.rope(np.array([1, 0, 0, 0], np.float32), 1, 4, c, s)
    assert out.tolist() == [c[0], s[0], 0.0, 0.0]
    out = o.rope(np.array([0, 1, 0, 0], np.float32), 1, 4, c, s)
    assert out.tolist() == [-s[0], c[0], 0.0, 0.0]
    rng = np.random.default_rng(33)
    x = rng.standard_normal(4 * 64).astype(np.float32)
    c, s = o.rope_table(517, 64)
    y = o.rope(x, 4, 64, c, s).astype(np.float64)
    n0 = x.reshape(-1, 2).astype(np.float64)
    assert np.allclose(np.hypot(*y.reshape(-1, 2).T), np.hypot(*n0.T), rtol=1e-6)
    q, k = rng.standard_normal(64).astype(np.float32), rng.standard_normal(64).astype(np.float32)
    def score(m, n):
        return float(np.dot(o.rope(q, 1, 64, *o.rope_table(m, 64)).astype(np.float64),
                            o.rope(k, 1, 64, *o.rope_table(n, 64)).astype(np.float64)))
    assert abs(score(10, 3) - score(107, 100)) < 1e-4 and abs(score(10, 3) - score(10, 4)) > 1e-3


def pin_attention(o):
    """One position returns its V row exactly; q = 0 averages the V rows;
    scores 0 and ln 3 weigh two rows 1/4 and 3/4; the tolerance scale
    sum_t p_t |V_t| takes the same weights over |V|; grouped heads equal
    multi-head attention over copied KV heads; the order of positions does
    not matter."""
    rng = np.random.default_rng(34)
    hd, nh, nkv = 8, 4, 2
    kc = rng.standard_normal((5, nkv * hd)).astype(np.float16).view(np.uint16)
    vc = rng.standard_normal((5, nkv * hd)).astype(np.float16).view(np.uint16)
    q = rng.standard_normal(nh * hd).astype(np.float32)
    out, absacc = o.attention(q, kc, vc, nh, nkv, hd, 1, nkv * hd)
    v0 = vc[0].view(np.float16).astype(np.float64)
    for h in range(nh):
        assert np.array_equal(out[h * hd:(h + 1) * hd], v0[(h // 2) * hd:(h // 2 + 1) * hd])
        # the tolerance scale sum_t p_t |V_t|: with one position, |V_0|
        assert np.array_equal(absacc[h * hd:(h + 1) * hd], np.abs(v0[(h // 2) * hd:(h // 2 + 1) * hd]))
    out, absacc = o.attention(np.zeros(nh * hd, np.float32), kc, vc, nh, nkv, hd, 5, nkv * hd)
    vm = vc.view(np.float16).astype(np.float64).mean(axis=0)
    vam = np.abs(vc.view(np.float16).astype(np.float64)).mean(axis=0)
    for h in range(nh):
        assert np.allclose(out[h * hd:(h + 1) * hd], vm[(h // 2) * hd:(h // 2 + 1) * hd], atol=1e-12)
        assert np.allclose(absacc[h * hd:(h + 1) * hd], vam[(h // 2) * hd:(h // 2 + 1) * hd], atol=1e-12)
    # two positions, one head of width 4: scores 0 and ln 3 (q scaled by
    # sqrt(4)), weights 1/4 and 3/4; the tolerance scale is 1/4 |V_0| + 3/4 |V_1|
    k2 = np.array([[0, 0, 0, 0], [1, 0, 0, 0]], np.float16).view(np.uint16)
    v2 = np.array([[4, 8, -2, 0], [8, 0, 2, 1]], np.float16).view(np.uint16)
    q2 = np.array([2 * np.log(3), 0, 0, 0], np.float32)
    out, absacc = o.attention(q2, k2, v2, 1, 1, 4, 2, 4)
    assert np.allclose(out, [7, 2, 1, 0.75], atol=1e-6)
    assert np.allclose(absacc, [7, 2, 2, 0.75], atol=1e-6)
    # grouped = multi-head with the KV heads copied
    kd = np.repeat(kc.reshape(5, nkv, hd), nh // nkv, axis=1).reshape(5, nh * hd)
    vd = np.repeat(vc.reshape(5, nkv, hd), nh // nkv, axis=1).reshape(5, nh * hd)
    a1, _ = o.attention(q, kc, vc, nh, nkv, hd, 5, nkv * hd)
    a2, _ = o.attention(q, kd, vd, nh, nh, hd, 5, nh * hd)
    assert np.array_equal(a1, a2)
    perm = [3, 0, 4, 1, 2]
    a3, _ = o.attention(q, kc[perm], vc[perm], nh, nkv, hd, 5, nkv * hd)
    assert np.allclose(a1, a3, rtol=1e-12, atol=1e-14)


def pin_swiglu(o):
    """silu(0) = 0, silu(ln 3) = (3/4) ln 3, silu(g) -> g for large g and
    -> 0 for very negative g; the up value multiplies."""
    g = np.array([0, np.log(3), 30, -30, -1], np.float32)
    u = np.array([5, 1, 2, 3, 1], np.float32)
    out = o.swiglu(g, u)
    assert out[0] == 0
    assert abs(out[1] - 0.75 * np.log(3)) < 1e-7  # g is ln 3 rounded to fp32
    assert abs(out[2] - 60) < 1e-9 and abs(out[3]) < 1e-11
    assert abs(out[4] - (-1 / (1 + np.e))) < 1e-15


def pin_quantize(o):
    """The encoder: inputs on the q8_0 grid (k * 2^-7, amax = 127 * 2^-7)
    come back as exactly k; points halfway between grid values round away
    from zero; the largest magnitude becomes +-127; every weight decodes to
    within half a step. q4_0 on hand values (the value of largest magnitude
    -8, so d = 1): code = min(15, trunc(x + 8.5)) and the -8 end decodes to
    itself."""
    k = np.arange(-127, 128)[:224].reshape(-1, 32).astype(np.float64)
    k[:, 0] = 127  # every block's largest magnitude is 127 * 2^-7, so d = 2^-7
    k[1, 1:] = np.arange(31) - 15 + 0.5  # halfway points
    x = (k.reshape(-1) * 2.0 ** -7).astype(np.float32)
    b = o.quantize(Q8_0, x).reshape(-1, 36)
    codes = b[:, 4:].view(np.int8).astype(np.int64).reshape(-1)
    assert np.all(b[:, :4].view(np.float32) == np.float32(2.0 ** -7))
    want = np.round(x.astype(np.float64) * 128)
    half = np.abs(x.astype(np.float64) * 128 - np.trunc(x.astype(np.float64) * 128)) == 0.5
    want[half] = np.trunc(x.astype(np.float64) * 128)[half] + np.sign(x[half])
    assert np.array_equal(codes, want.astype(np.int64))
    rng = np.random.default_rng(35)
    xr = (rng.standard_normal(32 * 64) * np.exp2(rng.integers(-10, 10, 32 * 64))).astype(np.float32)
    br = o.quantize(Q8_0, xr)
    w = o.dequantize_row(Q8_0, br, xr.size).astype(np.float64)
    d = np.repeat(br.reshape(-1, 36)[:, :4].copy().view(np.float32).reshape(-1).astype(np.float64), 32)
    assert np.all(np.abs(w - xr) <= d * (0.5 + 1e-5))
    am = np.abs(xr.reshape(-1, 32)).argmax(axis=1)
    cr = br.reshape(-1, 36)[:, 4:].view(np.int8)
    assert np.all(np.abs(cr[np.arange(len(am)), am]) == 127)
    # q4_0 hand values (d = 1): trunc(x + 8.5), capped at 15
    xs = np.array([-8, 7.4, 7.6, -7.5, 0.49, 0.5, -0.5, 3.2] + [0] * 24, np.float32)
    b4 = o.quantize(Q4_0, xs)
    assert b4[:2].view(np.float16)[0] == 1.0
    nib = np.concatenate([b4[2:] & 15, b4[2:] >> 4]).astype(np.int64)
    assert nib[:8].tolist() == [0, 15, 15, 1, 8, 9, 8, 11] and np.all(nib[8:] == 8)
    xr4 = rng.standard_normal(32 * 64).astype(np.float32)
    b4r = o.quantize(Q4_0, xr4)
    w4 = o.dequantize_row(Q4_0, b4r, xr4.size).astype(np.float64)
    d4 = np.abs(np.repeat(b4r.reshape(-1, 18)[:, :2].copy().view(np.float16).reshape(-1).astype(np.float64), 32))
    # half a step, except at the top end, where codes stop at 15 (+7 steps
    # against the -8 of the largest magnitude): up to one step there
    top = xr4.astype(np.float64) / -np.repeat(np.abs(xr4.reshape(-1, 32)).max(axis=1) *
                                              np.sign(xr4.reshape(-1, 32)[np.arange(64), np.abs(
                                                  xr4.reshape(-1, 32)).argmax(axis=1)]), 32) * 8 > 7.5
    assert np.all(np.abs(w4 - xr4) <= d4 * np.where(top, 1.0, 0.5) + np.abs(xr4) * 2e-3)
    mi = np.abs(xr4.reshape(-1, 32)).argmax(axis=1)
    assert np.allclose(w4.reshape(-1, 32)[np.arange(64), mi], xr4.reshape(-1, 32)[np.arange(64), mi], rtol=1e-3)


STEP_PINS = [pin_float_to_half, pin_rmsnorm, pin_rope, pin_attention, pin_swiglu, pin_quantize]
ALL_PINS += STEP_PINS


def failing_pins(o) -> list[str]:
    bad = []
    for p in ALL_PINS:
        try:
            p(o)
        except (AssertionError, ValueError):
            bad.append(p.__name__)
    return bad
