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
Q8_0_F16, Q5_1, Q5_K, Q2_K, Q3_K = 5, 6, 7, 8, 9
TYPES = {"q4_0": Q4_0, "q8_0": Q8_0, "Q4_K": Q4_K, "Q6_K": Q6_K, "Q8_0_F16": Q8_0_F16, "Q5_1": Q5_1, "Q5_K": Q5_K,
         "Q2_K": Q2_K, "Q3_K": Q3_K}

QK_OK, QK_EINVAL_TYPE, QK_EINVAL_SHAPE, QK_EINVAL_PTR, QK_EALIGN, QK_EHIP = 0, -1, -2, -3, -4, -5
QK_EIO, QK_EFORMAT, QK_ENOTFOUND, QK_ENOMEM = -6, -7, -8, -9

class QkGemvDesc(ctypes.Structure):
    """struct qk_gemv_desc of include/qk.h."""
    _fields_ = [("type", ctypes.c_int), ("W", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("cols", ctypes.c_int64), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p)]


class QkGemvInput(ctypes.Structure):
    """struct qk_gemv_input of include/qk_step.h."""
    _fields_ = [("kind", ctypes.c_int), ("aux", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("x_out", ctypes.c_void_p)]


QK_INPUT_PLAIN, QK_INPUT_ADD_RMSNORM, QK_INPUT_SWIGLU = 0, 1, 2
# qk_gemv_kernel_path results
QK_PATH_GENERIC, QK_PATH_FUSED, QK_PATH_STREAMED, QK_PATH_WIDE = 0, 1, 2, 3
# qk_gemm_kernel_path results
QK_GEMM_PATH_ROWS, QK_GEMM_PATH_FEW, QK_GEMM_PATH_PREFILL = 0, 3, 4
# qk_set_tuning keys
(QK_TUNE_GEMV_STREAM, QK_TUNE_GEMV_WGS_PER_CU, QK_TUNE_GEMV_SLOT, QK_TUNE_GEMV_NWR, QK_TUNE_GEMM_PATH,
 QK_TUNE_GEMM_KSPLIT, QK_TUNE_FEW_ROWS, QK_TUNE_FEW_KSW, QK_TUNE_FEW_DEPTH, QK_TUNE_PREFILL_TOKENS) = range(10)
TUNE_KEYS = {"gemv_stream": QK_TUNE_GEMV_STREAM, "gemv_wgs_per_cu": QK_TUNE_GEMV_WGS_PER_CU,
             "gemv_slot": QK_TUNE_GEMV_SLOT, "gemv_nwr": QK_TUNE_GEMV_NWR, "gemm_path": QK_TUNE_GEMM_PATH,
             "gemm_ksplit": QK_TUNE_GEMM_KSPLIT, "few_rows": QK_TUNE_FEW_ROWS, "few_ksw": QK_TUNE_FEW_KSW,
             "few_depth": QK_TUNE_FEW_DEPTH, "prefill_tokens": QK_TUNE_PREFILL_TOKENS}


class QkGemvPassInput(ctypes.Structure):
    """struct qk_gemv_pass_input of include/qk.h."""
    _fields_ = [("kind", ctypes.c_int), ("aux", ctypes.c_void_p), ("norm_w", ctypes.c_void_p),
                ("eps", ctypes.c_float)]


QK_PASS_IN_PLAIN, QK_PASS_IN_RMSNORM, QK_PASS_IN_SWIGLU = 0, 1, 2


class QkGgufTensor(ctypes.Structure):
    """struct qk_gguf_tensor of include/qk_gguf.h."""
    _fields_ = [("name", ctypes.c_char_p), ("n_dims", ctypes.c_int), ("dims", ctypes.c_int64 * 4),
                ("ggml_type", ctypes.c_int), ("qk_type", ctypes.c_int), ("offset", ctypes.c_int64),
                ("nbytes", ctypes.c_int64), ("data", ctypes.c_void_p)]


# Every symbol include/*.h declares, with (restype, argtypes).
_vp, _i64, _i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_pp = ctypes.POINTER(ctypes.c_void_p)
_cpp = ctypes.POINTER(ctypes.c_char_p)
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
    "qk_last_hip_error": (ctypes.c_char_p, []),
    "qk_set_tuning": (_i32, [_i32, _i32]),
    "qk_get_tuning": (_i32, [_i32]),
    "qk_probe_read": (_i32, [_vp, _i64, _vp, _i64, _vp]),
    "qk_probe_copy": (_i32, [_vp, _vp, _i64, _vp]),
    "qk_rmsnorm": (_i32, [_vp, _vp, _i64, ctypes.c_float, _vp, _vp]),
    "qk_add_rmsnorm": (_i32, [_vp, _vp, _vp, _i64, ctypes.c_float, _vp, _vp]),
    "qk_rope_tables": (_i32, [_i64, _i32, ctypes.c_double, _vp, _vp, _vp]),
    "qk_rope_kv": (_i32, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _i64, _vp]),
    "qk_attention_workspace_bytes": (_i64, [_i32, _i32, _i64]),
    "qk_attention": (_i32, [_vp, _vp, _vp, _vp, _i64, _i32, _i32, _i32, _i64, _vp, _i64, _vp, _vp]),
    "qk_attention_rope": (_i32, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _i64, _vp, _i64,
                                 _vp, _vp]),
    "qk_attention_scratch_limit": (_i64, []),
    "qk_attention_rope_noalloc": (_i32, [_vp, _vp, _vp, _vp, _i64, _vp, _vp, _i32, _i32, _i32, _vp, _vp, _i64, _vp,
                                         _vp]),
    "qk_swiglu": (_i32, [_vp, _vp, _i64, _vp, _vp]),
    "qk_quantize_row": (_i32, [_i32, _vp, _i64, _vp, _vp]),
    "qk_gemv_input_supported": (_i32, [_i32, _i64, _i64]),
    "qk_gemv_kernel_path": (_i32, [_i32, _i64, _i64]),
    "qk_gemv_pass_workspace_bytes": (_i64, [_vp, _i32, _vp, _vp]),
    "qk_gemv_pass_create": (_i32, [_vp, _i32, _vp, _vp, _vp, _i64, _pp]),
    "qk_gemv_pass_run": (_i32, [_vp, _vp]),
    "qk_gemv_pass_set_spin_limit": (_i32, [_vp, _i64]),
    "qk_gemv_pass_gave_up": (_i32, [_vp]),
    "qk_gemv_pass_grid": (_i32, [_vp]),
    "qk_gemv_pass_destroy": (None, [_vp]),
    "qk_gemm_kernel_path": (_i32, [_i32, _i64, _i64, _i64]),
    "qk_gemv_batch_input": (_i32, [_vp, _i32, _vp, _vp]),
    "qk_gguf_open": (_i32, [ctypes.c_char_p, _pp]),
    "qk_gguf_close": (None, [_vp]),
    "qk_gguf_version": (_i32, [_vp]),
    "qk_gguf_alignment": (_i64, [_vp]),
    "qk_gguf_tensor_count": (_i64, [_vp]),
    "qk_gguf_kv_count": (_i64, [_vp]),
    "qk_gguf_tensor_info": (_i32, [_vp, _i64, ctypes.POINTER(QkGgufTensor)]),
    "qk_gguf_find_tensor": (_i64, [_vp, ctypes.c_char_p]),
    "qk_gguf_find_key": (_i64, [_vp, ctypes.c_char_p]),
    "qk_gguf_key": (_i32, [_vp, _i64, _cpp, ctypes.POINTER(_i32)]),
    "qk_gguf_get_int": (_i32, [_vp, _i64, ctypes.POINTER(_i64)]),
    "qk_gguf_get_float": (_i32, [_vp, _i64, ctypes.POINTER(ctypes.c_double)]),
    "qk_gguf_get_string": (_i32, [_vp, _i64, _cpp, ctypes.POINTER(_i64)]),
    "qk_gguf_get_array": (_i32, [_vp, _i64, ctypes.POINTER(_i32), ctypes.POINTER(_i64), _pp]),
    "qk_gguf_get_array_string": (_i32, [_vp, _i64, _i64, _cpp, ctypes.POINTER(_i64)]),
    "qk_gguf_upload": (_i32, [_vp, _i64, _vp, _vp]),
}


class QkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib.qk_strerror(status).decode()
        detail = lib.qk_last_hip_error().decode()
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


def qk_set_tuning(key: int, value: int) -> int:
    """Sets a dispatch-table override (-1: the table's own choice); returns
    the previous value."""
    r = lib.qk_set_tuning(key, value)
    if r < -1:
        _check(r, "qk_set_tuning")
    return r


def qk_get_tuning(key: int) -> int:
    r = lib.qk_get_tuning(key)
    if r < -1:
        _check(r, "qk_get_tuning")
    return r


class tuning:
    """Context manager: `with tuning(gemm_path=QK_GEMM_PATH_FEW, few_ksw=3):`
    sets the named overrides (None leaves a key as it is) and restores the
    previous values on exit."""

    def __init__(self, **kw):
        self.kw = {TUNE_KEYS[k]: v for k, v in kw.items() if v is not None}
        self.prev = {}

    def __enter__(self):
        for k, v in self.kw.items():
            self.prev[k] = qk_set_tuning(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.prev.items():
            qk_set_tuning(k, v)
        return False


def qk_gemv(type: int, W, rows: int, cols: int, x, y, stream=None) -> None:
    """y[:rows] = W x, W given as packed blocks (device memory)."""
    _check(lib.qk_gemv(type, _ptr(W), rows, cols, _ptr(x), _ptr(y), _stream(stream)), "qk_gemv")


# ---- the decode step around the GEMVs (include/qk_step.h)

def qk_rmsnorm(x, w, n: int, eps: float, out, stream=None) -> None:
    _check(lib.qk_rmsnorm(_ptr(x), _ptr(w), n, eps, _ptr(out), _stream(stream)), "qk_rmsnorm")


def qk_add_rmsnorm(x, r, w, n: int, eps: float, out, stream=None) -> None:
    """x += r in place, then out = RMSNorm(x) * w."""
    _check(lib.qk_add_rmsnorm(_ptr(x), _ptr(r), _ptr(w), n, eps, _ptr(out), _stream(stream)), "qk_add_rmsnorm")


def qk_rope_tables(max_pos: int, head_dim: int, base: float, cos_table, sin_table, stream=None) -> None:
    _check(lib.qk_rope_tables(max_pos, head_dim, base, _ptr(cos_table), _ptr(sin_table), _stream(stream)),
           "qk_rope_tables")


def qk_rope_kv(q, k, v, pos, max_pos: int, cos_table, sin_table, n_heads: int, n_kv_heads: int, head_dim: int,
               k_cache, v_cache, kv_stride: int, stream=None) -> None:
    """pos: a device int32 tensor holding the position."""
    _check(lib.qk_rope_kv(_ptr(q), _ptr(k), _ptr(v), _ptr(pos), max_pos, _ptr(cos_table), _ptr(sin_table), n_heads,
                          n_kv_heads, head_dim, _ptr(k_cache), _ptr(v_cache), kv_stride, _stream(stream)),
           "qk_rope_kv")


def qk_attention_workspace_bytes(n_heads: int, head_dim: int, max_pos: int) -> int:
    return lib.qk_attention_workspace_bytes(n_heads, head_dim, max_pos)


def qk_attention(q, k_cache, v_cache, pos, max_pos: int, n_heads: int, n_kv_heads: int, head_dim: int,
                 kv_stride: int, workspace, out, stream=None) -> None:
    """workspace: a device tensor of at least qk_attention_workspace_bytes()."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.qk_attention(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(pos), max_pos, n_heads, n_kv_heads,
                            head_dim, kv_stride, _ptr(workspace), nbytes, _ptr(out), _stream(stream)),
           "qk_attention")


def qk_attention_rope(q, k, v, pos, max_pos: int, cos_table, sin_table, n_heads: int, n_kv_heads: int,
                      head_dim: int, k_cache, v_cache, kv_stride: int, workspace, out, stream=None) -> None:
    """RoPE, the fp16 cache store and attention in one call (q, k, v as
    projected)."""
    nbytes = workspace.numel() * workspace.element_size()
    _check(lib.qk_attention_rope(_ptr(q), _ptr(k), _ptr(v), _ptr(pos), max_pos, _ptr(cos_table), _ptr(sin_table),
                                 n_heads, n_kv_heads, head_dim, _ptr(k_cache), _ptr(v_cache), kv_stride,
                                 _ptr(workspace), nbytes, _ptr(out), _stream(stream)), "qk_attention_rope")


def qk_attention_rope_noalloc(q, k, v, pos, max_pos: int, cos_table, sin_table, n_heads: int, n_kv_heads: int,
                              head_dim: int, k_cache, v_cache, kv_stride: int, out, stream=None) -> None:
    """qk_attention_rope with the library's static per-GPU scratch instead of
    a workspace (allocates nothing; calls that overlap on one GPU race)."""
    _check(lib.qk_attention_rope_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(pos), max_pos, _ptr(cos_table),
                                         _ptr(sin_table), n_heads, n_kv_heads, head_dim, _ptr(k_cache),
                                         _ptr(v_cache), kv_stride, _ptr(out), _stream(stream)),
           "qk_attention_rope_noalloc")


def qk_swiglu(gate, up, n: int, out, stream=None) -> None:
    _check(lib.qk_swiglu(_ptr(gate), _ptr(up), n, _ptr(out), _stream(stream)), "qk_swiglu")


class GemvPass:
    """A persistent decode pass (qk_gemv_pass_*): `stages` is a list of
    stages, each a list of (type, W, rows, cols, x, y) GEMVs sharing one
    width and one x; `inputs` is None (every x used as it is) or one entry per
    stage: None, or (kind, aux, norm_w, eps) with kind QK_PASS_IN_*. An x or
    aux that is an earlier stage's y tensor chains the stages. The workspace
    is a device tensor this object owns; the tensors named in the stages and
    inputs must stay alive while it is used."""

    def __init__(self, stages, inputs=None):
        flat = [g for st in stages for g in st]
        ids = [i for i, st in enumerate(stages) for _ in st]
        self.descs = make_gemv_batch(flat)
        self.stage = (ctypes.c_int * len(ids))(*ids)
        self.inputs = None
        if inputs is not None:
            self.inputs = (QkGemvPassInput * len(stages))()
            for s, e in enumerate(inputs):
                if e is None:
                    self.inputs[s] = QkGemvPassInput(QK_PASS_IN_PLAIN, None, None, 0.0)
                else:
                    kind, aux, norm_w, eps = e
                    self.inputs[s] = QkGemvPassInput(kind, _ptr(aux), _ptr(norm_w), eps)
        ip = ctypes.addressof(self.inputs) if self.inputs is not None else None
        nbytes = lib.qk_gemv_pass_workspace_bytes(ctypes.addressof(self.descs), len(flat), self.stage, ip)
        if nbytes < 0:
            _check(nbytes, "qk_gemv_pass_workspace_bytes")
        self.workspace = torch.empty(nbytes + 256, dtype=torch.uint8, device="cuda")
        off = (-self.workspace.data_ptr()) % 256
        self.ws_ptr = self.workspace.data_ptr() + off
        self.handle = ctypes.c_void_p()
        _check(lib.qk_gemv_pass_create(ctypes.addressof(self.descs), len(flat), self.stage, ip, self.ws_ptr, nbytes,
                                       ctypes.byref(self.handle)), "qk_gemv_pass_create")

    def run(self, stream=None) -> None:
        _check(lib.qk_gemv_pass_run(self.handle, _stream(stream)), "qk_gemv_pass_run")

    def set_spin_limit(self, polls: int) -> None:
        _check(lib.qk_gemv_pass_set_spin_limit(self.handle, polls), "qk_gemv_pass_set_spin_limit")

    def gave_up(self) -> bool:
        r = lib.qk_gemv_pass_gave_up(self.handle)
        if r < 0:
            _check(r, "qk_gemv_pass_gave_up")
        return bool(r)

    @property
    def grid(self) -> int:
        return lib.qk_gemv_pass_grid(self.handle)

    def close(self) -> None:
        if self.handle:
            lib.qk_gemv_pass_destroy(self.handle)
            self.handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def qk_gemv_kernel_path(type: int, rows: int, cols: int) -> int:
    """QK_PATH_GENERIC / _FUSED / _STREAMED / _WIDE: the kernel qk_gemv runs
    for this format and shape (host-side; raises QkError on a bad type or
    shape)."""
    r = lib.qk_gemv_kernel_path(type, rows, cols)
    if r < 0:
        _check(r, "qk_gemv_kernel_path")
    return r


def qk_gemm_kernel_path(type: int, rows: int, cols: int, M: int) -> int:
    """QK_GEMM_PATH_*: the kernel qk_gemm_prefill runs for this format,
    shape and M (host-side; raises QkError on a bad type or shape)."""
    r = lib.qk_gemm_kernel_path(type, rows, cols, M)
    if r < 0:
        _check(r, "qk_gemm_kernel_path")
    return r


def qk_gemv_input_supported(type: int, rows: int, cols: int) -> bool:
    return bool(lib.qk_gemv_input_supported(type, rows, cols))


def make_gemv_input(kind: int, aux=None, norm_w=None, eps: float = 0.0, x_out=None) -> QkGemvInput:
    return QkGemvInput(kind, _ptr(aux), _ptr(norm_w), eps, _ptr(x_out))


def qk_gemv_batch_input(descs, inp: QkGemvInput, n: int | None = None, stream=None) -> None:
    """1-4 GEMVs sharing cols and x, with x transformed by `inp` inside the
    GEMV kernel (see include/qk_step.h). `descs` as for qk_gemv_batch."""
    if not isinstance(descs, ctypes.Array):
        descs = make_gemv_batch(descs)
    if n is None:
        n = getattr(descs, "n", len(descs))
    _check(lib.qk_gemv_batch_input(ctypes.addressof(descs), n, ctypes.byref(inp), _stream(stream)),
           "qk_gemv_batch_input")


def qk_quantize_row(type: int, x, n: int, blocks, stream=None) -> None:
    """The encoder: n fp32 values -> n/32 q8_0 or q4_0 blocks."""
    _check(lib.qk_quantize_row(type, _ptr(x), n, _ptr(blocks), _stream(stream)), "qk_quantize_row")


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


# ------------------------------------------------------------------ GGUF files

GGUF_SCALAR = {0: "B", 1: "b", 2: "H", 3: "h", 4: "I", 5: "i", 6: "f", 7: "?", 10: "Q", 11: "q", 12: "d"}


class GgufFile:
    """A GGUF file opened with qk_gguf_open (include/qk_gguf.h): the index,
    the metadata and uploads of tensor bytes to device memory. Marshalling
    only: the parsing is the library's."""

    def __init__(self, path: str):
        h = ctypes.c_void_p()
        _check(lib.qk_gguf_open(os.fsencode(path), ctypes.byref(h)), "qk_gguf_open")
        self._h = h

    def close(self) -> None:
        if self._h:
            lib.qk_gguf_close(self._h)
            self._h = ctypes.c_void_p()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def version(self) -> int:
        return lib.qk_gguf_version(self._h)

    @property
    def alignment(self) -> int:
        return lib.qk_gguf_alignment(self._h)

    def tensors(self) -> list[dict]:
        out = []
        for i in range(lib.qk_gguf_tensor_count(self._h)):
            t = QkGgufTensor()
            _check(lib.qk_gguf_tensor_info(self._h, i, ctypes.byref(t)), "qk_gguf_tensor_info")
            out.append({"index": i, "name": t.name.decode(), "dims": list(t.dims[:t.n_dims]),
                        "ggml_type": t.ggml_type, "qk_type": t.qk_type, "offset": t.offset, "nbytes": t.nbytes,
                        "data": t.data})
        return out

    def tensor(self, name: str) -> dict:
        i = lib.qk_gguf_find_tensor(self._h, name.encode())
        _check(int(i) if i < 0 else 0, f"qk_gguf_find_tensor({name})")
        return self.tensors()[i]

    def metadata(self) -> dict:
        out = {}
        for i in range(lib.qk_gguf_kv_count(self._h)):
            key, vt = ctypes.c_char_p(), ctypes.c_int()
            _check(lib.qk_gguf_key(self._h, i, ctypes.byref(key), ctypes.byref(vt)), "qk_gguf_key")
            out[key.value.decode()] = self._value(i, vt.value)
        return out

    def _value(self, i: int, vt: int):
        if vt in (6, 12):
            v = ctypes.c_double()
            _check(lib.qk_gguf_get_float(self._h, i, ctypes.byref(v)), "qk_gguf_get_float")
            return v.value
        if vt == 8:
            sp, n = ctypes.c_char_p(), ctypes.c_int64()
            _check(lib.qk_gguf_get_string(self._h, i, ctypes.byref(sp), ctypes.byref(n)), "qk_gguf_get_string")
            return ctypes.string_at(sp, n.value).decode("utf-8", "replace")
        if vt == 9:
            et, n, data = ctypes.c_int(), ctypes.c_int64(), ctypes.c_void_p()
            _check(lib.qk_gguf_get_array(self._h, i, ctypes.byref(et), ctypes.byref(n), ctypes.byref(data)),
                   "qk_gguf_get_array")
            if et.value == 8:
                vals = []
                for j in range(n.value):
                    sp, ln = ctypes.c_char_p(), ctypes.c_int64()
                    _check(lib.qk_gguf_get_array_string(self._h, i, j, ctypes.byref(sp), ctypes.byref(ln)),
                           "qk_gguf_get_array_string")
                    vals.append(ctypes.string_at(sp, ln.value).decode("utf-8", "replace"))
                return vals
            import struct
            fmt = GGUF_SCALAR[et.value]
            raw = ctypes.string_at(data, n.value * struct.calcsize("<" + fmt)) if n.value else b""
            return list(struct.unpack("<%d%s" % (n.value, fmt), raw))
        v = ctypes.c_int64()
        _check(lib.qk_gguf_get_int(self._h, i, ctypes.byref(v)), "qk_gguf_get_int")
        return bool(v.value) if vt == 7 else v.value

    def upload(self, name: str, dst, stream=None) -> None:
        """Copies the tensor's bytes into the device tensor dst (uint8,
        at least nbytes) on torch's current stream (or `stream`)."""
        t = self.tensor(name)
        if dst.numel() * dst.element_size() < t["nbytes"]:
            raise ValueError(f"{name}: destination holds fewer than {t['nbytes']} bytes")
        _check(lib.qk_gguf_upload(self._h, t["index"], _ptr(dst), _stream(stream)), "qk_gguf_upload")
