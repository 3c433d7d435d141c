"""Thin ctypes binding of libqk.so (include/qk.h).

Argument marshalling only: torch tensors become device pointers, the stream
defaults to torch's current stream, and a non-zero status raises QkError.
Every step of the computation runs in the library's HIP kernels; there is no
Python or CPU fallback. If the library is missing or fails to load, import
fails loudly.

torch is imported before the library is loaded so that the library binds to
the HIP runtime torch already loaded (both carry the SONAME libamdhip64.so.7).
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (must precede loading libqk.so)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqk.so")

Q4_0, Q8_0, Q4_K, Q6_K = 1, 2, 3, 4
TYPES = {"q4_0": Q4_0, "q8_0": Q8_0, "Q4_K": Q4_K, "Q6_K": Q6_K}

QK_OK, QK_EINVAL_TYPE, QK_EINVAL_SHAPE, QK_EINVAL_PTR, QK_EALIGN, QK_EHIP = 0, -1, -2, -3, -4, -5

class QkGemvDesc(ctypes.Structure):
    """struct qk_gemv_desc of include/qk.h."""
    _fields_ = [("type", ctypes.c_int), ("W", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


# Every symbol include/qk.h declares, with (restype, argtypes).
_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
SIGNATURES = {
    "qk_block_elems": (_i32, [_i32]),
    "qk_block_bytes": (_i32, [_i32]),
    "qk_row_bytes": (_i64, [_i32, _i64]),
    "qk_dequantize_row": (_i32, [_i32, _vp, _i64, _vp]),
    "qk_dequantize_row_async": (_i32, [_i32, _vp, _i64, _vp, _vp]),
    "qk_gemv": (_i32, [_i32, _vp, _i64, _i64, _vp, _vp, _vp]),
    "qk_gemm_prefill": (_i32, [_i32, _vp, _i64, _i64, _vp, _i64, _vp, _vp]),
    "qk_gemv_batch": (_i32, [_vp, _i32, _vp]),
    "qk_strerror": (ctypes.c_char_p, [_i32]),
    "qk_last_error": (ctypes.c_char_p, []),
    "qk_probe_read": (_i32, [_vp, _i64, _vp, _i64, _vp]),
    "qk_probe_copy": (_i32, [_vp, _vp, _i64, _vp]),
}


class QkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.qk_strerror(status).decode()
        detail = lib.qk_last_error().decode()
        super().__init__(f"{where}: {msg} ({status}){': ' + detail if detail else ''}")


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"libqk.so not built at {path}; run block_quantized_weight_gemv_amd/build.py")
    l = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(l, name)
        fn.restype = res
        fn.argtypes = args
    return l


lib = _load()


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream) -> int | None:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(torch.cuda.current_device())
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != QK_OK:
        raise QkError(status, where)


def qk_block_elems(type: int) -> int:
    return lib.qk_block_elems(type)


def qk_block_bytes(type: int) -> int:
    return lib.qk_block_bytes(type)


def qk_row_bytes(type: int, cols: int) -> int:
    return lib.qk_row_bytes(type, cols)


def qk_dequantize_row(type: int, blocks, n: int, out, stream=None) -> None:
    """out[:n] = fp32 weights of the blocks (bit-exact). With stream=None the
    call is enqueued on torch's current stream (qk_dequantize_row_async); pass
    stream=0 for the library's null-stream entry point."""
    if stream == 0:
        _check(lib.qk_dequantize_row(type, _ptr(blocks), n, _ptr(out)), "qk_dequantize_row")
    else:
        _check(lib.qk_dequantize_row_async(type, _ptr(blocks), n, _ptr(out), _stream(stream)),
               "qk_dequantize_row_async")


def qk_gemv(type: int, W, rows: int, cols: int, x, y, stream=None) -> None:
    """y[:rows] = W x, W given as packed blocks (device memory)."""
    _check(lib.qk_gemv(type, _ptr(W), rows, cols, _ptr(x), _ptr(y), _stream(stream)), "qk_gemv")


def make_gemv_batch(items) -> "ctypes.Array":
    """items: iterable of (type, W, rows, cols, x, y); returns the descriptor
    array for qk_gemv_batch (build it once and reuse it in a loop)."""
    items = list(items)
    arr = (QkGemvDesc * max(len(items), 1))()
    for i, (t, W, r, c, x, y) in enumerate(items):
        arr[i] = QkGemvDesc(t, _ptr(W), r, c, _ptr(x), _ptr(y))
    arr.n = len(items)
    return arr


def qk_gemv_batch(descs, n: int | None = None, stream=None) -> None:
    """Independent GEMVs in as few launches as possible. `descs` is an array
    from make_gemv_batch or a list of (type, W, rows, cols, x, y) tuples."""
    if not isinstance(descs, ctypes.Array):
        descs = make_gemv_batch(descs)
    if n is None:
        n = getattr(descs, "n", len(descs))
    _check(lib.qk_gemv_batch(ctypes.addressof(descs), n, _stream(stream)), "qk_gemv_batch")


def qk_gemm_prefill(type: int, W, rows: int, cols: int, X, M: int, Y, stream=None) -> None:
    """Y[M, rows] = X W^T with X bfloat16 [M, cols] (tensor of dtype bfloat16
    or int16/uint16 bit patterns), Y fp32."""
    _check(lib.qk_gemm_prefill(type, _ptr(W), rows, cols, _ptr(X), M, _ptr(Y), _stream(stream)),
           "qk_gemm_prefill")


def qk_probe_read(buf, nbytes: int, out, stream=None) -> None:
    """Streaming-read probe over buf[:nbytes] (see include/qk_probe.h)."""
    st = lib.qk_probe_read(_ptr(buf), nbytes, _ptr(out), out.numel(), _stream(stream))
    if st != 0:
        raise RuntimeError(f"qk_probe_read failed ({st})")


def qk_probe_copy(src, dst, nbytes: int, stream=None) -> None:
    """Plain copy of nbytes from src to dst (see include/qk_probe.h)."""
    st = lib.qk_probe_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream))
    if st != 0:
        raise RuntimeError(f"qk_probe_copy failed ({st})")

