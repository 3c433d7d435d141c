"""The C-ABI library on the CPU: it loads, exports every function
include/qk.h declares, answers the table queries, and rejects every invalid
argument with its status code before touching a GPU (no compute call
reaches HIP in this file)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include"))) if h.endswith(".h")]


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(qk_[a-z_0-9]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def qk():
    from block_quantized_weight_gemv_amd import qk as mod

    return mod


def test_header_declares_the_hot_calls():
    names = declared_functions()
    for f in ("qk_dequantize_row", "qk_gemv", "qk_gemm_prefill"):
        assert f in names


def test_library_exports_every_declared_symbol(qk):
    for name in declared_functions():
        assert hasattr(qk.lib, name), name
        assert name in qk.SIGNATURES, f"binding lacks a prototype for {name}"


def test_format_table(qk):
    assert [qk.qk_block_elems(t) for t in (qk.Q4_0, qk.Q8_0, qk.Q4_K, qk.Q6_K)] == [32, 32, 256, 256]
    assert [qk.qk_block_bytes(t) for t in (qk.Q4_0, qk.Q8_0, qk.Q4_K, qk.Q6_K)] == [18, 36, 144, 210]
    assert qk.qk_row_bytes(qk.Q4_K, 2048) == 8 * 144
    assert qk.qk_row_bytes(qk.Q6_K, 5632) == 22 * 210
    assert qk.qk_row_bytes(qk.Q8_0, 64) == 72
    assert qk.qk_row_bytes(qk.Q4_0, 0) == 0
    new = (qk.Q8_0_F16, qk.Q5_1, qk.Q5_K, qk.Q2_K, qk.Q3_K)
    assert [qk.qk_block_elems(t) for t in new] == [32, 32, 256, 256, 256]
    assert [qk.qk_block_bytes(t) for t in new] == [34, 24, 176, 84, 110]
    assert qk.qk_row_bytes(qk.Q2_K, 5632) == 22 * 84
    for bad in (0, 10, -1, 99):
        assert qk.qk_block_elems(bad) == qk.QK_EINVAL_TYPE
        assert qk.qk_block_bytes(bad) == qk.QK_EINVAL_TYPE
        assert qk.qk_row_bytes(bad, 256) == qk.QK_EINVAL_TYPE
    assert qk.qk_row_bytes(qk.Q4_K, 100) == qk.QK_EINVAL_SHAPE
    assert qk.qk_row_bytes(qk.Q4_0, -32) == qk.QK_EINVAL_SHAPE


def test_strerror(qk):
    for st in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9):
        assert qk.lib.qk_strerror(st) != b"unknown status"
    assert qk.lib.qk_strerror(-100) == b"unknown status"


def test_last_hip_error_names_the_failed_check(qk):
    """qk_last_hip_error (and its shorter alias qk_last_error) holds the
    message of the calling thread's last failed call."""
    assert qk.lib.qk_gemv(qk.Q4_K, None, 4, 256, A16, A16, None) == qk.QK_EINVAL_PTR
    assert qk.lib.qk_last_hip_error() == b"W is NULL"
    assert qk.lib.qk_last_error() == qk.lib.qk_last_hip_error()
    assert qk.lib.qk_gemv(qk.Q4_K, A16, 4, 256, A16, A16 + 2, None) == qk.QK_EALIGN
    assert b"y" in qk.lib.qk_last_hip_error()


def test_tuning_overrides(qk):
    """qk_set_tuning / qk_get_tuning: every key starts at -1 (the table's own
    choice), takes a value and gives back the previous one; unknown keys and
    values below -1 are QK_EINVAL_SHAPE; the context manager restores."""
    for k in range(10):
        assert qk.qk_get_tuning(k) == -1
    assert qk.lib.qk_set_tuning(qk.QK_TUNE_FEW_KSW, 3) == -1
    assert qk.qk_get_tuning(qk.QK_TUNE_FEW_KSW) == 3
    assert qk.lib.qk_set_tuning(qk.QK_TUNE_FEW_KSW, -1) == 3
    assert qk.lib.qk_set_tuning(10, 1) == qk.QK_EINVAL_SHAPE
    assert qk.lib.qk_set_tuning(-1, 1) == qk.QK_EINVAL_SHAPE
    assert qk.lib.qk_set_tuning(0, -2) == qk.QK_EINVAL_SHAPE
    assert qk.lib.qk_get_tuning(10) == qk.QK_EINVAL_SHAPE
    with qk.tuning(gemm_path=qk.QK_GEMM_PATH_ROWS, gemv_stream=1):
        assert qk.qk_get_tuning(qk.QK_TUNE_GEMM_PATH) == 0 and qk.qk_get_tuning(qk.QK_TUNE_GEMV_STREAM) == 1
        assert qk.qk_gemm_kernel_path(qk.Q4_K, 64, 2048, 512) == qk.QK_GEMM_PATH_ROWS
    assert qk.qk_get_tuning(qk.QK_TUNE_GEMM_PATH) == -1 and qk.qk_get_tuning(qk.QK_TUNE_GEMV_STREAM) == -1


A16 = 0x10000  # a fake, 16-byte aligned address: never dereferenced, the checks fail first


def test_gemv_argument_errors(qk):
    g = qk.lib.qk_gemv
    assert g(17, A16, 4, 256, A16, A16, None) == qk.QK_EINVAL_TYPE
    assert g(qk.Q4_K, A16, -1, 256, A16, A16, None) == qk.QK_EINVAL_SHAPE
    assert g(qk.Q4_K, A16, 4, -256, A16, A16, None) == qk.QK_EINVAL_SHAPE
    assert g(qk.Q4_K, A16, 4, 100, A16, A16, None) == qk.QK_EINVAL_SHAPE  # ragged: not whole blocks
    assert g(qk.Q4_0, A16, 4, 48, A16, A16, None) == qk.QK_EINVAL_SHAPE
    assert g(qk.Q4_K, None, 4, 256, A16, A16, None) == qk.QK_EINVAL_PTR
    assert g(qk.Q4_K, A16, 4, 256, None, A16, None) == qk.QK_EINVAL_PTR
    assert g(qk.Q4_K, A16, 4, 256, A16, None, None) == qk.QK_EINVAL_PTR
    assert g(qk.Q4_K, A16 + 4, 4, 256, A16, A16, None) == qk.QK_EALIGN
    assert g(qk.Q4_K, A16, 4, 256, A16 + 8, A16, None) == qk.QK_EALIGN
    assert g(qk.Q4_K, A16, 4, 256, A16, A16 + 2, None) == qk.QK_EALIGN
    assert g(qk.Q6_K, A16, 1 << 62, 1 << 20, A16, A16, None) == qk.QK_EINVAL_SHAPE  # size overflow
    assert b"W" in qk.lib.qk_last_error() or qk.lib.qk_last_error()
    # empty matrix: nothing to do, nothing launched, pointers may be NULL
    assert g(qk.Q4_K, None, 0, 256, None, None, None) == qk.QK_OK
    assert g(qk.Q6_K, None, 0, 0, None, None, None) == qk.QK_OK
    # y must not overlap W (4 rows of 144 bytes) or x (256 floats): a
    # workgroup that starts late would stage an x that y has overwritten
    X = A16 + 0x1000
    assert g(qk.Q4_K, A16, 4, 256, X, A16 + 0x100, None) == qk.QK_EINVAL_PTR
    assert g(qk.Q4_K, A16, 4, 256, X, X, None) == qk.QK_EINVAL_PTR          # in place
    assert g(qk.Q4_K, A16, 4, 256, X, X + 1020, None) == qk.QK_EINVAL_PTR   # y's first float is x's last
    assert g(qk.Q4_K, A16, 4, 256, X, X - 12, None) == qk.QK_EINVAL_PTR     # y's last float is x's first
    assert b"overlaps" in qk.lib.qk_last_hip_error()


def test_dequant_argument_errors(qk):
    d = qk.lib.qk_dequantize_row_async
    assert d(0, A16, 256, A16, None) == qk.QK_EINVAL_TYPE
    assert d(qk.Q6_K, A16, 100, A16, None) == qk.QK_EINVAL_SHAPE
    assert d(qk.Q6_K, A16, -256, A16, None) == qk.QK_EINVAL_SHAPE
    assert d(qk.Q6_K, None, 256, A16, None) == qk.QK_EINVAL_PTR
    assert d(qk.Q6_K, A16, 256, None, None) == qk.QK_EINVAL_PTR
    assert d(qk.Q6_K, A16 + 2, 256, A16, None) == qk.QK_EALIGN
    assert d(qk.Q6_K, A16, 256, A16 + 1, None) == qk.QK_EALIGN
    assert d(qk.Q8_0, None, 0, None, None) == qk.QK_OK
    assert qk.lib.qk_dequantize_row(qk.Q4_K, None, 0, None) == qk.QK_OK
    assert qk.lib.qk_dequantize_row(19, A16, 256, A16) == qk.QK_EINVAL_TYPE


def test_gemm_argument_errors(qk):
    g = qk.lib.qk_gemm_prefill
    assert g(-3, A16, 4, 256, A16, 2, A16, None) == qk.QK_EINVAL_TYPE
    assert g(qk.Q4_K, A16, 4, 256, A16, -1, A16, None) == qk.QK_EINVAL_SHAPE
    assert g(qk.Q4_K, A16, 4, 96, A16, 2, A16, None) == qk.QK_EINVAL_SHAPE
    assert g(qk.Q4_K, A16, 4, 256, None, 2, A16, None) == qk.QK_EINVAL_PTR
    assert g(qk.Q4_K, A16, 4, 256, A16, 2, None, None) == qk.QK_EINVAL_PTR
    assert g(qk.Q4_K, A16, 4, 256, A16 + 8, 2, A16, None) == qk.QK_EALIGN
    assert g(qk.Q4_K, A16, 4, 256, A16, 2, A16 + 2, None) == qk.QK_EALIGN
    assert g(qk.Q4_K, None, 4, 256, None, 0, None, None) == qk.QK_OK  # M = 0
    assert g(qk.Q4_K, None, 0, 256, None, 5, None, None) == qk.QK_OK  # rows = 0
    # Y must not overlap W (4 rows of 144 bytes) or X (2 x 256 bf16)
    X = A16 + 0x1000
    assert g(qk.Q4_K, A16, 4, 256, X, 2, A16 + 0x100, None) == qk.QK_EINVAL_PTR
    assert g(qk.Q4_K, A16, 4, 256, X, 2, X + 0x200, None) == qk.QK_EINVAL_PTR
    assert g(qk.Q4_K, A16, 4, 256, X, 2, X - 16, None) == qk.QK_EINVAL_PTR  # Y's 32 bytes reach X


def test_binding_raises(qk):
    with pytest.raises(qk.QkError) as e:
        qk.qk_gemv(99, A16, 4, 256, A16, A16, stream=0)
    assert e.value.status == qk.QK_EINVAL_TYPE
    with pytest.raises(qk.QkError):
        qk.qk_dequantize_row(qk.Q4_K, A16, 17, A16, stream=0)


def test_gemv_batch_argument_errors(qk):
    b = qk.lib.qk_gemv_batch
    assert b(None, 0, None) == qk.QK_OK
    assert b(None, -1, None) == qk.QK_EINVAL_SHAPE
    assert b(None, 2, None) == qk.QK_EINVAL_PTR
    good = (qk.Q4_K, A16, 4, 256, A16 + 0x1000, A16 + 0x2000)
    for bad, status in [((19, A16, 4, 256, A16, A16 + 0x2000), qk.QK_EINVAL_TYPE),
                        ((qk.Q4_K, A16, 4, 100, A16, A16 + 0x2000), qk.QK_EINVAL_SHAPE),
                        ((qk.Q4_K, None, 4, 256, A16, A16 + 0x2000), qk.QK_EINVAL_PTR),
                        ((qk.Q4_K, A16 + 4, 4, 256, A16 + 0x1000, A16 + 0x2000), qk.QK_EALIGN),
                        ((qk.Q6_K, A16 + 0x8000, 4, 256, A16 + 0x1000, A16 + 0x2004), qk.QK_EINVAL_PTR)]:
        arr = qk.make_gemv_batch([good, bad])
        st = b(qk.ctypes.addressof(arr), 2, None)
        assert st == status, (bad, st)
    # an output overlapping an input (its own W) is rejected before any launch
    arr = qk.make_gemv_batch([(qk.Q4_K, A16, 4, 256, A16 + 0x1000, A16 + 8)])
    assert b(qk.ctypes.addressof(arr), 1, None) == qk.QK_EINVAL_PTR
    # empty descriptors only: nothing to launch
    arr = qk.make_gemv_batch([(qk.Q4_K, None, 0, 256, None, None), (qk.Q6_K, None, 0, 0, None, None)])
    assert b(qk.ctypes.addressof(arr), 2, None) == qk.QK_OK


def test_probe_argument_errors(qk):
    """The measurement probes reject bad arguments before launching anything."""
    lib = qk.lib
    assert lib.qk_probe_copy(None, 4096, 64, None) == -1
    assert lib.qk_probe_copy(4096, 8192, 24, None) == -1   # not a multiple of 16
    assert lib.qk_probe_copy(4096, 4104, 64, None) == -1   # misaligned dst
    assert lib.qk_probe_copy(4096, 4112, 64, None) == -1   # overlapping buffers
    assert lib.qk_probe_read(None, 64, 4096, 8, None) == -1
    assert lib.qk_probe_read(4096, 0, 8192, 8, None) == -1


def test_step_argument_errors(qk):
    """The decode-step calls reject bad arguments on the host, before any
    HIP call (no GPU needed)."""
    L = qk.lib
    assert L.qk_rmsnorm(None, A16, 8, 1e-5, A16, None) == qk.QK_EINVAL_PTR
    assert L.qk_rmsnorm(A16, A16, 0, 1e-5, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_rmsnorm(A16, A16, 65537, 1e-5, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_add_rmsnorm(A16, A16, A16, 8, 1e-5, A16, None) == qk.QK_EINVAL_PTR  # out aliases x
    assert L.qk_rope_tables(0, 64, 1e4, A16, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_rope_tables(16, 63, 1e4, A16, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_rope_tables(16, 64, -1.0, A16, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_rope_kv(A16, A16, A16, A16, 16, A16, A16, 32, 5, 64, A16, A16, 320, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_rope_kv(A16, A16, A16, A16, 16, A16, A16, 32, 4, 64, A16, A16, 255, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_rope_kv(A16, A16, A16, None, 16, A16, A16, 32, 4, 64, A16, A16, 256, None) == qk.QK_EINVAL_PTR
    ws = L.qk_attention_workspace_bytes(32, 64, 2048)
    assert ws == 32 * 32 * 66 * 4  # one (max, sum, 64 weighted V sums) state per head and 64-position chunk
    # chunks grow past 16384 rows so that there are at most 256 of them
    assert L.qk_attention_workspace_bytes(2, 128, 16384) == 2 * 256 * 130 * 4
    assert L.qk_attention_workspace_bytes(2, 128, 16385) == 2 * 129 * 130 * 4
    assert L.qk_attention_workspace_bytes(2, 128, 65536) == 2 * 256 * 130 * 4
    assert L.qk_attention_workspace_bytes(2, 128, 65537) == qk.QK_EINVAL_SHAPE
    assert L.qk_attention(A16, A16, A16, A16, 2048, 32, 4, 96, 256, A16, ws, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_attention(A16, A16 + 8, A16, A16, 2048, 32, 4, 64, 256, A16, ws, A16, None) == qk.QK_EALIGN
    assert L.qk_attention(A16, A16, A16, A16, 2048, 32, 4, 64, 260, A16, ws, A16, None) == qk.QK_EALIGN
    assert L.qk_attention(A16, A16, A16, A16, 2048, 32, 4, 64, 256, A16, ws - 4, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_attention(A16, A16, A16, A16, 2048, 32, 4, 64, 256, None, ws, A16, None) == qk.QK_EINVAL_PTR
    # the call without a workspace: sizes past its static scratch and null
    # pointers are rejected before any HIP call
    assert L.qk_attention_scratch_limit() == 8 << 20
    assert L.qk_attention_rope_noalloc(A16, A16, A16, A16, 65536, A16, A16, 65, 5, 128, A16, A16, 640, A16,
                                       None) == qk.QK_EINVAL_SHAPE
    assert L.qk_attention_rope_noalloc(A16, A16, A16, A16, 2048, A16, A16, 32, 4, 96, A16, A16, 384, A16,
                                       None) == qk.QK_EINVAL_SHAPE
    assert L.qk_attention_rope_noalloc(A16, None, A16, A16, 2048, A16, A16, 32, 4, 64, A16, A16, 256, A16,
                                       None) == qk.QK_EINVAL_PTR
    assert L.qk_swiglu(None, A16, 8, A16, None) == qk.QK_EINVAL_PTR
    assert L.qk_swiglu(A16, A16, -1, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_quantize_row(qk.Q4_K, A16, 256, A16, None) == qk.QK_EINVAL_TYPE
    assert L.qk_quantize_row(qk.Q8_0, A16, 33, A16, None) == qk.QK_EINVAL_SHAPE
    assert L.qk_quantize_row(qk.Q8_0, A16 + 4, 32, A16, None) == qk.QK_EALIGN
    assert L.qk_quantize_row(qk.Q4_0, A16, 0, None, None) == qk.QK_OK


def test_gemv_batch_input_argument_errors(qk):
    import ctypes

    L = qk.lib
    d = (qk.QkGemvDesc * 2)()
    d[0] = qk.QkGemvDesc(qk.Q4_K, A16, 4, 2048, A16 + 0x100000, A16 + 0x200000)
    d[1] = qk.QkGemvDesc(qk.Q4_K, A16 + 0x300000, 4, 2048, A16 + 0x100000, A16 + 0x400000)
    plain = qk.QkGemvInput(0, None, None, 0.0, None)
    ok_norm = qk.QkGemvInput(1, A16 + 0x500000, A16 + 0x600000, 1e-5, A16 + 0x700000)
    ref = ctypes.addressof
    assert L.qk_gemv_batch_input(ref(d), 0, ctypes.byref(plain), None) == qk.QK_EINVAL_SHAPE
    assert L.qk_gemv_batch_input(ref(d), 5, ctypes.byref(plain), None) == qk.QK_EINVAL_SHAPE
    assert L.qk_gemv_batch_input(ref(d), 1, None, None) == qk.QK_EINVAL_PTR
    assert L.qk_gemv_batch_input(ref(d), 1, ctypes.byref(qk.QkGemvInput(3, None, None, 0.0, None)),
                                 None) == qk.QK_EINVAL_TYPE
    assert L.qk_gemv_batch_input(ref(d), 1, ctypes.byref(qk.QkGemvInput(1, A16, None, 0.0, A16)),
                                 None) == qk.QK_EINVAL_PTR
    assert L.qk_gemv_batch_input(ref(d), 1, ctypes.byref(qk.QkGemvInput(2, None, None, 0.0, None)),
                                 None) == qk.QK_EINVAL_PTR
    assert L.qk_gemv_batch_input(ref(d), 1, ctypes.byref(qk.QkGemvInput(2, A16 + 4, None, 0.0, None)),
                                 None) == qk.QK_EALIGN
    bad = qk.QkGemvInput(1, A16 + 0x500000, A16 + 0x600000, 1e-5, A16 + 0x100000)  # x_out = x
    assert L.qk_gemv_batch_input(ref(d), 1, ctypes.byref(bad), None) == qk.QK_EINVAL_PTR
    d2 = (qk.QkGemvDesc * 2)()
    d2[0] = d[0]
    d2[1] = qk.QkGemvDesc(qk.Q4_K, A16 + 0x300000, 4, 2048, A16 + 0x800000, A16 + 0x400000)  # another x
    assert L.qk_gemv_batch_input(ref(d2), 2, ctypes.byref(ok_norm), None) == qk.QK_EINVAL_SHAPE
    d3 = (qk.QkGemvDesc * 1)()
    d3[0] = qk.QkGemvDesc(qk.Q5_K, A16, 4, 2048, A16 + 0x100000, A16 + 0x200000)  # no transformed-input kernel
    assert L.qk_gemv_batch_input(ref(d3), 1, ctypes.byref(ok_norm), None) == qk.QK_EINVAL_SHAPE


def test_gemv_pass_argument_errors(qk):
    """qk_gemv_pass_create checks the stages, the formats and shapes, the
    inputs (each an earlier stage's whole output or memory apart from every
    output), the input transforms, the output overlaps and the workspace
    before any HIP call; qk_gemv_pass_workspace_bytes runs the same checks
    and counts a mirror for every output that a later stage reads."""
    import ctypes

    L = qk.lib
    MB = 1 << 20
    x0, x1 = A16 + 100 * MB, A16 + 101 * MB
    aux0, nw0 = A16 + 102 * MB, A16 + 103 * MB

    def desc(t, w, rows, cols, x, y):
        return (t, A16 + w * MB, rows, cols, x, A16 + 200 * MB + y * MB)

    Y0 = A16 + 200 * MB  # the first output's y
    good = [desc(qk.Q4_K, 0, 2048, 2048, x0, 0), desc(qk.Q6_K, 1, 256, 2048, x0, 1),
            desc(qk.Q4_K, 2, 2048, 2048, Y0, 2)]  # stage 1 reads stage 0's first y
    h = ctypes.c_void_p()

    def arrays(items, stage, inputs):
        arr = qk.make_gemv_batch(items)
        st = (ctypes.c_int * len(stage))(*stage)
        ins = None
        if inputs is not None:
            ins = (qk.QkGemvPassInput * len(inputs))(*[qk.QkGemvPassInput(*e) for e in inputs])
        return arr, st, ins

    def wsbytes(items, stage, inputs=None):
        arr, st, ins = arrays(items, stage, inputs)
        return L.qk_gemv_pass_workspace_bytes(ctypes.addressof(arr), len(items), st,
                                              ctypes.addressof(ins) if ins is not None else None)

    ws_bytes = wsbytes(good, [0, 0, 1])
    assert ws_bytes > 0
    # one chained output of 2048 rows: 2048 mirror words of 8 bytes
    assert ws_bytes - wsbytes([good[0], good[1], desc(qk.Q4_K, 2, 2048, 2048, x1, 2)], [0, 0, 1]) == 8 * 2048
    assert L.qk_gemv_pass_workspace_bytes(None, 1, None, None) == qk.QK_EINVAL_PTR
    assert wsbytes(good, [0, 0, 2]) == qk.QK_EINVAL_SHAPE

    def create(items, stage, inputs=None, ws=A16 + 400 * MB, nbytes=ws_bytes):
        arr, st, ins = arrays(items, stage, inputs)
        return L.qk_gemv_pass_create(ctypes.addressof(arr), len(items), st,
                                     ctypes.addressof(ins) if ins is not None else None, ws, nbytes, ctypes.byref(h))

    assert L.qk_gemv_pass_create(None, 1, None, None, A16, 0, None) == qk.QK_EINVAL_PTR
    assert create(good, [1, 1, 2]) == qk.QK_EINVAL_SHAPE          # stages start at 0
    assert create(good, [0, 0, 2]) == qk.QK_EINVAL_SHAPE          # and rise by 0 or 1
    assert create(good, [0, 1, 0]) == qk.QK_EINVAL_SHAPE
    five = [desc(qk.Q4_K, i, 64, 2048, x0, i) for i in range(5)]
    assert create(five, [0] * 5) == qk.QK_EINVAL_SHAPE             # at most 4 GEMVs per stage
    assert create([good[0], desc(qk.Q4_K, 1, 64, 2048, x1, 1)], [0, 0]) == qk.QK_EINVAL_SHAPE  # one x per stage
    assert create([good[0], desc(qk.Q4_K, 1, 64, 4096, x0, 1)], [0, 0]) == qk.QK_EINVAL_SHAPE  # one width
    assert create([desc(qk.Q8_0, 0, 64, 2048, x0, 0)], [0]) == qk.QK_EINVAL_SHAPE   # Q4_K / Q6_K only
    assert create([desc(qk.Q4_K, 0, 64, 8192, x0, 0)], [0]) == qk.QK_EINVAL_SHAPE   # up to 6144 columns
    assert create([desc(qk.Q4_K, 0, 0, 2048, x0, 0)], [0]) == qk.QK_EINVAL_SHAPE    # rows needed
    assert create([desc(qk.Q4_K, 0, 64, 2048, x0, 0), desc(qk.Q4_K, 1, 64, 2048, x0, 0)],
                  [0, 0]) == qk.QK_EINVAL_PTR                                        # outputs overlap
    assert create([(qk.Q4_K, A16, 64, 2048, x0, A16 + 1024)], [0]) == qk.QK_EINVAL_PTR  # output over W
    # inputs: an earlier stage's whole output, or apart from every output
    assert create([(qk.Q4_K, A16, 64, 2048, x0, x0 + 4096)], [0]) == qk.QK_EINVAL_PTR   # x over its own output
    assert b"earlier stage's whole output" in L.qk_last_hip_error()
    assert create([good[0], good[1], desc(qk.Q4_K, 2, 2048, 2048, Y0 + 16, 2)],
                  [0, 0, 1]) == qk.QK_EINVAL_PTR                                     # part of an output
    assert create([good[0], good[1], desc(qk.Q4_K, 2, 2048, 2048, A16 + 201 * MB, 2)],
                  [0, 0, 1]) == qk.QK_EINVAL_PTR                                     # 256 rows as 2048 columns
    assert create([desc(qk.Q4_K, 0, 2048, 2048, A16 + 201 * MB, 0), desc(qk.Q4_K, 1, 2048, 2048, x0, 1)],
                  [0, 1]) == qk.QK_EINVAL_PTR                                        # a later stage's output
    plain = (qk.QK_PASS_IN_PLAIN, None, None, 0.0)
    assert create(good, [0, 0, 1], [plain, (7, None, None, 0.0)]) == qk.QK_EINVAL_SHAPE    # unknown kind
    assert create(good, [0, 0, 1], [plain, (qk.QK_PASS_IN_SWIGLU, None, None, 0.0)]) == qk.QK_EINVAL_PTR
    assert create(good, [0, 0, 1], [plain, (qk.QK_PASS_IN_SWIGLU, aux0 + 4, None, 0.0)]) == qk.QK_EALIGN
    assert create(good, [0, 0, 1], [plain, (qk.QK_PASS_IN_SWIGLU, Y0 + 16, None, 0.0)]) == qk.QK_EINVAL_PTR
    assert create(good, [0, 0, 1], [plain, (qk.QK_PASS_IN_RMSNORM, None, None, 0.0)]) == qk.QK_EINVAL_SHAPE
    assert create(good, [0, 0, 1], [plain, (qk.QK_PASS_IN_RMSNORM, None, None, -1.0)]) == qk.QK_EINVAL_SHAPE
    assert create(good, [0, 0, 1], [plain, (qk.QK_PASS_IN_RMSNORM, None, nw0 + 8, 1e-5)]) == qk.QK_EALIGN
    assert create(good, [0, 0, 1], [plain, (qk.QK_PASS_IN_RMSNORM, None, Y0, 1e-5)]) == qk.QK_EINVAL_PTR
    # the workspace
    assert create(good, [0, 0, 1], ws=None) == qk.QK_EINVAL_PTR
    assert create(good, [0, 0, 1], ws=A16 + 400 * MB + 16) == qk.QK_EALIGN
    assert create(good, [0, 0, 1], nbytes=ws_bytes - 8) == qk.QK_EINVAL_SHAPE
    assert create(good, [0, 0, 1], ws=Y0) == qk.QK_EINVAL_PTR                          # over an output
    assert L.qk_gemv_pass_run(None, None) == qk.QK_EINVAL_PTR
    assert L.qk_gemv_pass_gave_up(None) == qk.QK_EINVAL_PTR
    assert L.qk_gemv_pass_set_spin_limit(None, 5) == qk.QK_EINVAL_PTR
    L.qk_gemv_pass_destroy(None)
