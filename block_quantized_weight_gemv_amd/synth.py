"""Seeded synthetic inputs: random block bytes, activation vectors and
bfloat16 activation matrices.

This module is shared by the tests, the smoke check and the benchmark, and
serves the GPU path and the CPU oracle alike. It holds none of the method's
arithmetic: it draws random bytes and random field values and writes each
field at its byte offset; it never decodes a block or multiplies anything.
fp16/fp32 field values are rounded by numpy's own casts.

Field distributions (the synthetic stand-ins for TinyLlama-1.1B Q4_K_M
weights, which the pages run but which are not available here):

* Q4_K (144 B): fp16 d and dmin uniform in [1e-3, 1e-2]; the 12 packed
  scale/min bytes uniform (all 96 bits are used exactly once by the eight
  6-bit scales and eight 6-bit mins, so uniform bytes are uniform 0..63
  fields); 128 nibble bytes uniform.
* Q6_K (210 B): ql/qh bytes uniform; int8 scales uniform in [-64, 63];
  fp16 d uniform in [1e-4, 1e-3].
* q8_0 (36 B): fp32 scale uniform in [1e-3, 2e-2]; int8 values uniform in
  [-127, 127].
* q4_0 (18 B): fp16 scale uniform in [1e-3, 2e-2]; 16 nibble bytes uniform.
* The ggml-layout formats, built the same way (uniform code, high-bit and
  scale bytes; uniform fp16 scales in the ranges of the formats above):
  Q8_0 with an fp16 scale (34 B): d in [1e-3, 2e-2], int8 in [-127, 127];
  Q5_1 (24 B): d in [1e-3, 2e-2], m in [-2e-2, 0]; Q5_K (176 B): d, dmin in
  [1e-3, 1e-2]; Q2_K (84 B): d, dmin in [1e-3, 1e-2]; Q3_K (110 B): d in
  [1e-3, 1e-2].
* x: fp32 N(0, 1). X: N(0, 1) rounded to bfloat16 (nearest-even).
* Full field range (`full=True`, for parity tests): every field over all the
  values its format can hold, not only the ranges above: Q6_K int8 scales
  uniform in [-128, 127]; q8_0 and Q8_0_F16 codes uniform in [-128, 127];
  fp16 scales (d, dmin, Q5_1's m) with a random sign, 1/8 of them subnormal
  (a random non-zero fraction), 1/32 of them zero of either sign, the rest
  of magnitude uniform in the format's range above; q8_0's fp32 scale with a
  random sign, 1/8 of them of magnitude 2^u with u uniform in [-140, -100]
  (below 2^-126 they are fp32 subnormals).
* The decode step's weights (step.py) use the same fields with the scale
  ranges multiplied by 0.02 (weights of magnitude ~0.02, as in a trained
  decoder, so that activations and attention scores stay of order one), and
  norm weights uniform in [0.5, 1.5].

Every stream is ``numpy.random.default_rng([seed, stream_id])`` (PCG64 under
a SeedSequence), so a (seed, stream) pair names its data on every machine.
"""
from __future__ import annotations

import numpy as np

Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K = 5, 6, 7, 8, 9
NAMES = {Q4_0: "q4_0", Q8_0: "q8_0", Q4_K: "Q4_K", Q6_K: "Q6_K", Q8_0_F16: "Q8_0_F16", Q5_1: "Q5_1", Q5_K: "Q5_K",
         Q2_K: "Q2_K", Q3_K: "Q3_K"}
BLOCK_ELEMS = {Q4_K: 256, Q6_K: 256, Q4_0: 32, Q8_0: 32, Q8_0_F16: 32, Q5_1: 32, Q5_K: 256, Q2_K: 256, Q3_K: 256}
BLOCK_BYTES = {Q4_K: 144, Q6_K: 210, Q4_0: 18, Q8_0: 36, Q8_0_F16: 34, Q5_1: 24, Q5_K: 176, Q2_K: 84, Q3_K: 110}


def rng(seed: int, stream: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream)])


def row_bytes(t: int, cols: int) -> int:
    return cols // BLOCK_ELEMS[t] * BLOCK_BYTES[t]


def _f16_bytes(vals: np.ndarray) -> np.ndarray:
    return vals.astype(np.float16).view(np.uint8).reshape(-1, 2)


def blocks(t: int, nblocks: int, g: np.random.Generator, scale: float = 1.0, full: bool = False) -> np.ndarray:
    """nblocks random blocks of format t as uint8[nblocks, block_bytes];
    `scale` multiplies the ranges of the block scales (and Q5_1's minimum),
    so the weights scale by it (the default gives the ranges above); `full`
    draws every field over its whole range (see the module notes)."""
    bb = BLOCK_BYTES[t]
    out = g.integers(0, 256, size=(nblocks, bb), dtype=np.uint8)

    def u(a, b):
        return g.uniform(a * scale, b * scale, nblocks)

    def f16(a, b):
        """fp16 scale bytes: magnitudes uniform in [a, b]; in full mode with
        random signs, subnormals and zeros."""
        h = u(a, b).astype(np.float16).view(np.uint16)
        if full:
            sign = g.integers(0, 2, nblocks).astype(np.uint16) << 15
            pick = g.random(nblocks)
            sub = g.integers(1, 0x400, nblocks).astype(np.uint16)
            h = np.where(pick < 1 / 32, 0, np.where(pick < 1 / 32 + 1 / 8, sub, h & 0x7FFF)).astype(np.uint16) | sign
        return h.view(np.uint8).reshape(-1, 2)

    def codes8():
        lo = -128 if full else -127
        return g.integers(lo, 128, size=(nblocks, 32), dtype=np.int8).view(np.uint8)

    if t == Q4_K:
        out[:, 0:2] = f16(1e-3, 1e-2)
        out[:, 2:4] = f16(1e-3, 1e-2)
    elif t == Q6_K:
        lo = -128 if full else -64
        out[:, 192:208] = g.integers(lo, 128 if full else 64, size=(nblocks, 16), dtype=np.int8).view(np.uint8)
        out[:, 208:210] = f16(1e-4, 1e-3)
    elif t == Q8_0:
        s = u(1e-3, 2e-2).astype(np.float32)
        if full:
            tiny = np.exp2(g.uniform(-140.0, -100.0, nblocks)).astype(np.float32)
            s = np.where(g.random(nblocks) < 1 / 8, tiny, s) * np.where(g.random(nblocks) < 0.5, -1, 1)
        out[:, 0:4] = s.astype(np.float32).view(np.uint8).reshape(-1, 4)
        out[:, 4:36] = codes8()
    elif t == Q4_0:
        out[:, 0:2] = f16(1e-3, 2e-2)
    elif t == Q8_0_F16:
        out[:, 0:2] = f16(1e-3, 2e-2)
        out[:, 2:34] = codes8()
    elif t == Q5_1:
        out[:, 0:2] = f16(1e-3, 2e-2)
        if full:
            out[:, 2:4] = f16(0.0, 2e-2)
        else:
            out[:, 2:4] = _f16_bytes(u(-2e-2, 0.0))
    elif t == Q5_K:
        out[:, 0:2] = f16(1e-3, 1e-2)
        out[:, 2:4] = f16(1e-3, 1e-2)
    elif t == Q2_K:
        out[:, 80:82] = f16(1e-3, 1e-2)
        out[:, 82:84] = f16(1e-3, 1e-2)
    elif t == Q3_K:
        out[:, 108:110] = f16(1e-3, 1e-2)
    else:
        raise ValueError(f"unknown format id {t}")
    return out


def matrix(t: int, rows: int, cols: int, seed: int, stream: int = 0, scale: float = 1.0,
           full: bool = False) -> np.ndarray:
    """A rows x cols weight matrix of format t: uint8[rows * row_bytes]."""
    if cols % BLOCK_ELEMS[t]:
        raise ValueError("cols must be a multiple of the block size")
    nb = rows * (cols // BLOCK_ELEMS[t])
    return blocks(t, nb, rng(seed, stream), scale, full).reshape(-1)


def vector(n: int, seed: int, stream: int = 1000) -> np.ndarray:
    """fp32 N(0, 1) activations."""
    return rng(seed, stream).standard_normal(n, dtype=np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (nearest, ties to even); returns the
    16-bit patterns. Inputs here are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_matrix(M: int, cols: int, seed: int, stream: int = 2000) -> np.ndarray:
    """bfloat16 N(0, 1) activations as uint16[M, cols]."""
    x = rng(seed, stream).standard_normal((M, cols), dtype=np.float32)
    return bf16_bits(x).reshape(M, cols)
