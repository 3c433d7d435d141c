"""CPU oracle for block-quantized weight decoding, GEMV and GEMM.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The GPU library
never calls it, and the two share no code: the arithmetic lives in
``qk_oracle.c`` (plain C11, fp32 decode in the pages' operation order, fp64
sums), built with gcc and loaded here through ctypes. This module only
marshals numpy arrays.

Parity pins: every function here is pinned by the ``-m "not gpu"`` tests
(hand-assembled blocks with hand-computed values, exact rational arithmetic,
library fp16 conversion, brute-force sums, mutation checks).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qk_oracle.c")
LIB = os.path.join(HERE, "libqk_oracle.so")

# Format ids, defined independently of the GPU library (same values).
Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K = 5, 6, 7, 8, 9
TYPES = {"q4_0": Q4_0, "q8_0": Q8_0, "Q4_K": Q4_K, "Q6_K": Q6_K, "Q8_0_F16": Q8_0_F16, "Q5_1": Q5_1,
         "Q5_K": Q5_K, "Q2_K": Q2_K, "Q3_K": Q3_K}

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(src: str = SRC, out: str = LIB, extra_flags: list[str] | None = None) -> str:
    """Compile the oracle with gcc into a shared library; returns its path."""
    cmd = ["gcc", *CFLAGS, *(extra_flags or []), "-o", out + ".tmp", src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes view of one built oracle library (the real one, or a mutant
    built by a test from an edited copy of the source)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            build(out=path)
        lib = ctypes.CDLL(path)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.qko_block_elems.argtypes = [i32]
        lib.qko_block_elems.restype = i32
        lib.qko_block_bytes.argtypes = [i32]
        lib.qko_block_bytes.restype = i32
        lib.qko_half_to_float.argtypes = [ctypes.c_uint16]
        lib.qko_half_to_float.restype = ctypes.c_float
        lib.qko_bf16_to_float.argtypes = [ctypes.c_uint16]
        lib.qko_bf16_to_float.restype = ctypes.c_float
        lib.qko_dequantize_row.argtypes = [i32, vp, i64, vp]
        lib.qko_dequantize_row.restype = i32
        lib.qko_gemv.argtypes = [i32, vp, i64, i64, vp, vp, vp]
        lib.qko_gemv.restype = i32
        lib.qko_gemm.argtypes = [i32, vp, i64, i64, vp, i64, vp, vp]
        lib.qko_gemm.restype = i32
        f32 = ctypes.c_float
        lib.qko_float_to_half.argtypes = [f32]
        lib.qko_float_to_half.restype = ctypes.c_uint16
        lib.qko_rmsnorm.argtypes = [vp, vp, i64, f32, vp]
        lib.qko_rmsnorm.restype = None
        lib.qko_rope_table.argtypes = [i64, i32, ctypes.c_double, vp, vp]
        lib.qko_rope_table.restype = None
        lib.qko_rope_interleaved.argtypes = [vp, i32, i32, vp, vp]
        lib.qko_rope_interleaved.restype = None
        lib.qko_attention.argtypes = [vp, vp, vp, i32, i32, i32, i64, i64, vp, vp]
        lib.qko_attention.restype = None
        lib.qko_swiglu.argtypes = [vp, vp, i64, vp]
        lib.qko_swiglu.restype = None
        lib.qko_quantize.argtypes = [i32, vp, i64, vp]
        lib.qko_quantize.restype = i32
        self.lib = lib
        self.path = path

    # -- scalars ---------------------------------------------------------
    def block_elems(self, t: int) -> int:
        return self.lib.qko_block_elems(t)

    def block_bytes(self, t: int) -> int:
        return self.lib.qko_block_bytes(t)

    def half_to_float(self, h: int) -> float:
        return self.lib.qko_half_to_float(h)

    def bf16_to_float(self, h: int) -> float:
        return self.lib.qko_bf16_to_float(h)

    def row_bytes(self, t: int, cols: int) -> int:
        return cols // self.block_elems(t) * self.block_bytes(t)

    # -- arrays ----------------------------------------------------------
    def dequantize_row(self, t: int, blocks: np.ndarray, n: int) -> np.ndarray:
        blocks = np.ascontiguousarray(blocks, dtype=np.uint8)
        out = np.empty(n, dtype=np.float32)
        need = n // max(self.block_elems(t), 1) * self.block_bytes(t)
        if blocks.nbytes < need:
            raise ValueError("not enough block bytes")
        rc = self.lib.qko_dequantize_row(t, blocks.ctypes.data, n, out.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle dequantize_row failed (type={t}, n={n})")
        return out

    def gemv(self, t: int, W: np.ndarray, rows: int, cols: int, x: np.ndarray):
        """Returns (y, absacc), both float64[rows]."""
        W = np.ascontiguousarray(W, dtype=np.uint8)
        x = np.ascontiguousarray(x, dtype=np.float32)
        if W.nbytes < rows * self.row_bytes(t, cols) or x.size < cols:
            raise ValueError("operand too small")
        y = np.empty(rows, dtype=np.float64)
        a = np.empty(rows, dtype=np.float64)
        rc = self.lib.qko_gemv(t, W.ctypes.data, rows, cols, x.ctypes.data, y.ctypes.data, a.ctypes.data)
        if rc != 0:
            raise ValueError(f"oracle gemv failed (type={t}, rows={rows}, cols={cols})")
        return y, a

    def gemv_rows(self, t: int, W: np.ndarray, cols: int, x: np.ndarray, row_ids):
        """Oracle GEMV on selected rows only (for sampled checks at full size)."""
        W = np.ascontiguousarray(W, dtype=np.uint8).reshape(-1)
        rb = self.row_bytes(t, cols)
        ys, As = [], []
        for r in row_ids:
            y, a = self.gemv(t, W[int(r) * rb:(int(r) + 1) * rb], 1, cols, x)
            ys.append(y[0])
            As.append(a[0])
        return np.array(ys), np.array(As)

    def gemm(self, t: int, W: np.ndarray, rows: int, cols: int, X_bf16: np.ndarray, M: int):
        """X_bf16: uint16[M, cols]. Returns (Y, absacc), float64[M, rows]."""
        W = np.ascontiguousarray(W, dtype=np.uint8)
        X = np.ascontiguousarray(X_bf16, dtype=np.uint16)
        if W.nbytes < rows * self.row_bytes(t, cols) or X.size < M * cols:
            raise ValueError("operand too small")
        Y = np.empty((M, rows), dtype=np.float64)
        A = np.empty((M, rows), dtype=np.float64)
        rc = self.lib.qko_gemm(t, W.ctypes.data, rows, cols, X.ctypes.data, M, Y.ctypes.data, A.ctypes.data)
        if rc != 0:
            raise ValueError("oracle gemm failed")
        return Y, A

    # -- the decode step around the GEMVs, and the encoder -----------------
    def float_to_half(self, v: float) -> int:
        return self.lib.qko_float_to_half(v)

    def halves(self, a) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float32).reshape(-1)
        return np.array([self.lib.qko_float_to_half(float(v)) for v in a], dtype=np.uint16)

    def rmsnorm(self, x, w, eps: float) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        out = np.empty_like(x)
        self.lib.qko_rmsnorm(x.ctypes.data, w.ctypes.data, x.size, eps, out.ctypes.data)
        return out

    def rope_table(self, pos: int, head_dim: int, base: float = 10000.0):
        c = np.empty(head_dim // 2, dtype=np.float32)
        s = np.empty(head_dim // 2, dtype=np.float32)
        self.lib.qko_rope_table(pos, head_dim, base, c.ctypes.data, s.ctypes.data)
        return c, s

    def rope(self, x, n_heads: int, head_dim: int, c, s) -> np.ndarray:
        out = np.array(x, dtype=np.float32, copy=True).reshape(-1)
        c = np.ascontiguousarray(c, dtype=np.float32)
        s = np.ascontiguousarray(s, dtype=np.float32)
        self.lib.qko_rope_interleaved(out.ctypes.data, n_heads, head_dim, c.ctypes.data, s.ctypes.data)
        return out

    def attention(self, q, kc, vc, n_heads: int, n_kv: int, head_dim: int, n_pos: int, kv_stride: int):
        """q fp32 [n_heads*head_dim]; kc/vc fp16 bit patterns (uint16), row t
        of head g at t*kv_stride + g*head_dim. Returns (out, absacc) fp64."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        kc = np.ascontiguousarray(kc, dtype=np.uint16)
        vc = np.ascontiguousarray(vc, dtype=np.uint16)
        if n_pos > 0 and kc.size < (n_pos - 1) * kv_stride + n_kv * head_dim:
            raise ValueError("cache too small")
        out = np.empty(n_heads * head_dim, dtype=np.float64)
        a = np.empty(n_heads * head_dim, dtype=np.float64)
        self.lib.qko_attention(q.ctypes.data, kc.ctypes.data, vc.ctypes.data, n_heads, n_kv, head_dim, n_pos,
                               kv_stride, out.ctypes.data, a.ctypes.data)
        return out, a

    def swiglu(self, g, u) -> np.ndarray:
        g = np.ascontiguousarray(g, dtype=np.float32)
        u = np.ascontiguousarray(u, dtype=np.float32)
        out = np.empty(g.size, dtype=np.float64)
        self.lib.qko_swiglu(g.ctypes.data, u.ctypes.data, g.size, out.ctypes.data)
        return out

    def quantize(self, t: int, x) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32).reshape(-1)
        out = np.zeros(x.size // 32 * self.block_bytes(t), dtype=np.uint8)
        if self.lib.qko_quantize(t, x.ctypes.data, x.size, out.ctypes.data) != 0:
            raise ValueError("oracle quantize failed")
        return out


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default


def within_tolerance(y_test, y_ref, absacc):
    """The pass rule for GEMV/GEMM outputs: |y - y_ref| <= 1e-4 * sum|w*x| + 1e-6,
    elementwise. Returns (ok, worst ratio of error to allowance)."""
    y_test = np.asarray(y_test, dtype=np.float64)
    allow = 1e-4 * np.asarray(absacc, dtype=np.float64) + 1e-6
    err = np.abs(y_test - np.asarray(y_ref, dtype=np.float64))
    ratio = err / allow
    bad = ~np.isfinite(y_test)
    worst = float(np.max(ratio)) if ratio.size else 0.0
    return bool(np.all(ratio <= 1.0) and not bad.any()), worst
