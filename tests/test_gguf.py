"""The GGUF reader (include/qk_gguf.h) on files the suite writes itself
(tests/gguf_writer.py): header, metadata of every value type, the tensor
index with absolute offsets and sizes, alignment, the mapped bytes, and
QK_EFORMAT (never a crash) for malformed files, including every truncation
of a valid one. Host-only: no GPU call."""
from __future__ import annotations

import ctypes
import os
import struct

import numpy as np
import pytest

import gguf_writer as gw


@pytest.fixture(scope="module")
def qk():
    from block_quantized_weight_gemv_amd import qk as mod

    return mod


def rand_bytes(n: int, seed: int) -> bytes:
    return np.random.default_rng(seed).integers(0, 256, n, dtype=np.uint8).tobytes()


KVS = [
    ("general.architecture", gw.STRING, "llama"),
    ("general.name", gw.STRING, "tiny synthetic é"),
    ("llama.block_count", gw.UINT32, 22),
    ("llama.context_length", gw.UINT64, 2048),
    ("llama.rope.freq_base", gw.FLOAT32, 10000.0),
    ("llama.attention.layer_norm_rms_epsilon", gw.FLOAT64, 1e-5),
    ("test.u8", gw.UINT8, 250), ("test.i8", gw.INT8, -7), ("test.u16", gw.UINT16, 65000),
    ("test.i16", gw.INT16, -30000), ("test.i32", gw.INT32, -123456), ("test.i64", gw.INT64, -(1 << 40)),
    ("test.bool", gw.BOOL, 1),
    ("tokenizer.ggml.tokens", gw.ARRAY, (gw.STRING, ["<unk>", "<s>", "</s>", "▁the", ""])),
    ("tokenizer.ggml.scores", gw.ARRAY, (gw.FLOAT32, [0.0, -1.5, 2.25])),
    ("tokenizer.ggml.token_type", gw.ARRAY, (gw.INT32, [2, 3, 3, 1, 1])),
    ("test.empty", gw.ARRAY, (gw.UINT32, [])),
]


def tensors(seed: int = 0):
    specs = [("blk.0.attn_q.weight", [512, 3], gw.Q4_K), ("blk.0.ffn_down.weight", [256, 5], gw.Q6_K),
             ("blk.0.attn_v.weight", [64, 4], gw.Q4_0), ("output_norm.weight", [7], gw.F32),
             ("token_embd.weight", [64, 2], gw.Q8_0), ("rope_freqs", [3, 5], gw.F16),
             ("blk.0.ffn_up.weight", [256, 2, 1], gw.Q5_K)]
    return [(n, d, t, rand_bytes(gw.tensor_bytes(d, t), seed + i)) for i, (n, d, t) in enumerate(specs)]


def write(tmp_path, blob: bytes, name: str = "m.gguf") -> str:
    p = os.path.join(tmp_path, name)
    with open(p, "wb") as fh:
        fh.write(blob)
    return p


@pytest.mark.parametrize("alignment,version", [(32, 3), (64, 3), (32, 2), (256, 3)])
def test_roundtrip(qk, tmp_path, alignment, version):
    kvs = list(KVS) + ([("general.alignment", gw.UINT32, alignment)] if alignment != 32 else [])
    ts = tensors(alignment)
    blob = gw.build(kvs, ts, version=version, alignment=alignment)
    with qk.GgufFile(write(tmp_path, blob)) as f:
        assert f.version == version and f.alignment == alignment
        meta = f.metadata()
        for k, t, v in kvs:
            got = meta[k]
            if t == gw.ARRAY:
                et, items = v
                if et == gw.FLOAT32:
                    assert got == pytest.approx(items)
                else:
                    assert got == items
            elif t == gw.FLOAT32:
                assert got == pytest.approx(v)
            elif t == gw.BOOL:
                assert got is bool(v)
            else:
                assert got == v, k
        got = f.tensors()
        assert [g["name"] for g in got] == [t[0] for t in ts]
        data0 = gw.data_start(blob, alignment)
        qk_types = {gw.Q4_K[0]: qk.Q4_K, gw.Q6_K[0]: qk.Q6_K, gw.Q4_0[0]: qk.Q4_0, gw.Q5_K[0]: qk.Q5_K,
                    gw.Q8_0[0]: qk.Q8_0_F16}  # GGUF's Q8_0 is the 34-byte fp16-scale block
        for g, (name, dims, gt, data) in zip(got, ts):
            assert g["dims"] == dims and g["ggml_type"] == gt[0]
            assert g["qk_type"] == qk_types.get(gt[0], 0)
            assert g["nbytes"] == len(data)
            assert g["offset"] % alignment == 0 and g["offset"] >= data0
            assert blob[g["offset"]:g["offset"] + g["nbytes"]] == data
            assert ctypes.string_at(g["data"], g["nbytes"]) == data  # the mapped bytes
        assert f.tensor("blk.0.ffn_down.weight")["dims"] == [256, 5]


def test_weight_matrix_layout_is_qk_layout(qk, tmp_path):
    """A matrix of `rows` outputs and `cols` inputs has dims {cols, rows} and
    its bytes are the rows of qk.h's W, back to back."""
    rows, cols = 6, 512
    from block_quantized_weight_gemv_amd import synth

    W = synth.matrix(qk.Q4_K, rows, cols, seed=3)
    blob = gw.build([], [("w", [cols, rows], gw.Q4_K, W.tobytes())])
    with qk.GgufFile(write(tmp_path, blob)) as f:
        t = f.tensor("w")
        assert t["nbytes"] == rows * qk.lib.qk_row_bytes(qk.Q4_K, cols)
        assert ctypes.string_at(t["data"], t["nbytes"]) == W.tobytes()


def test_find_and_types(qk, tmp_path):
    blob = gw.build(KVS, tensors())
    p = write(tmp_path, blob)
    with qk.GgufFile(p) as f:
        h = f._h
        lib = qk.lib
        assert lib.qk_gguf_find_tensor(h, b"nope") == qk.QK_ENOTFOUND
        assert lib.qk_gguf_find_key(h, b"nope") == qk.QK_ENOTFOUND
        i = lib.qk_gguf_find_key(h, b"general.name")
        v = ctypes.c_int64()
        assert lib.qk_gguf_get_int(h, i, ctypes.byref(v)) == qk.QK_EINVAL_TYPE  # a string, not an int
        d = ctypes.c_double()
        assert lib.qk_gguf_get_float(h, lib.qk_gguf_find_key(h, b"test.i32"), ctypes.byref(d)) == qk.QK_EINVAL_TYPE
        t = qk.QkGgufTensor()
        assert lib.qk_gguf_tensor_info(h, 99, ctypes.byref(t)) == qk.QK_ENOTFOUND
        assert lib.qk_gguf_tensor_info(h, -1, ctypes.byref(t)) == qk.QK_ENOTFOUND
        s, n = ctypes.c_char_p(), ctypes.c_int64()
        j = lib.qk_gguf_find_key(h, b"tokenizer.ggml.tokens")
        assert lib.qk_gguf_get_array_string(h, j, 5, ctypes.byref(s), ctypes.byref(n)) == qk.QK_ENOTFOUND
        assert lib.qk_gguf_get_array_string(h, j, 3, ctypes.byref(s), ctypes.byref(n)) == qk.QK_OK
        assert ctypes.string_at(s, n.value).decode() == "▁the"
    assert qk.lib.qk_gguf_version(None) == qk.QK_EINVAL_PTR
    qk.lib.qk_gguf_close(None)  # no-op


def status_of(qk, path: str) -> int:
    h = ctypes.c_void_p()
    s = qk.lib.qk_gguf_open(os.fsencode(path), ctypes.byref(h))
    if s == qk.QK_OK:
        qk.lib.qk_gguf_close(h)
    else:
        assert not h.value  # nothing handed out on failure
    return s


def test_open_errors(qk, tmp_path):
    assert status_of(qk, os.path.join(tmp_path, "missing.gguf")) == qk.QK_EIO
    assert status_of(qk, write(tmp_path, b"", "empty.gguf")) == qk.QK_EFORMAT
    good = gw.build(KVS, tensors())
    assert status_of(qk, write(tmp_path, good)) == qk.QK_OK
    bad = {
        "magic": gw.build(KVS, tensors(), magic=b"GGML"),
        "version1": gw.build(KVS, tensors(), version=1),
        "version4": gw.build(KVS, tensors(), version=4),
        "bool2": gw.build([("b", gw.BOOL, 2)], []),
        "unknown value type": gw.build([], [])[:16] + struct.pack("<Q", 1) + gw.gstr("k") + struct.pack("<I", 13),
        "alignment not pow2": gw.build([("general.alignment", gw.UINT32, 48)], [], alignment=48),
        "alignment wrong type": gw.build([("general.alignment", gw.UINT64, 32)], []),
        "duplicate key": gw.build([("a", gw.UINT8, 1), ("a", gw.UINT8, 2)], []),
        "duplicate tensor": gw.build([], [("t", [32], gw.F32, bytes(128)), ("t", [32], gw.F32, bytes(128))]),
    }
    for name, blob in bad.items():
        assert status_of(qk, write(tmp_path, blob, "bad.gguf")) == qk.QK_EFORMAT, name


def patch_tensor_info(blob: bytes, field: str, val: int, index: int = 0) -> bytes:
    """Rewrites one field of tensor info `index` in a file build() wrote."""
    b = bytearray(blob)
    pos = 8
    nt, nkv = struct.unpack_from("<QQ", b, pos)
    pos += 16
    assert nkv == 0
    for i in range(nt):
        (n,) = struct.unpack_from("<Q", b, pos)
        pos += 8 + n
        (nd,) = struct.unpack_from("<I", b, pos)
        if i == index:
            if field == "n_dims":
                struct.pack_into("<I", b, pos, val)
            elif field == "dim0":
                struct.pack_into("<Q", b, pos + 4, val)
            elif field == "type":
                struct.pack_into("<I", b, pos + 4 + 8 * nd, val)
            elif field == "offset":
                struct.pack_into("<Q", b, pos + 4 + 8 * nd + 4, val)
            return bytes(b)
        pos += 4 + 8 * nd + 12
    raise AssertionError("no such tensor")


def test_index_errors(qk, tmp_path):
    ts = [("a", [256, 2], gw.Q4_K, rand_bytes(288, 1)), ("b", [64], gw.F32, rand_bytes(256, 2))]
    good = gw.build([], ts)
    assert status_of(qk, write(tmp_path, good)) == qk.QK_OK
    cases = {
        "offset not aligned": patch_tensor_info(good, "offset", 8, 1),
        "data past the end": patch_tensor_info(good, "offset", 1 << 20, 1),
        "offset overflows": patch_tensor_info(good, "offset", (1 << 64) - 32, 1),
        "unknown type": patch_tensor_info(good, "type", 99, 0),
        "cols not whole blocks": patch_tensor_info(good, "dim0", 100, 0),
        "zero dimension": patch_tensor_info(good, "dim0", 0, 0),
        "huge dimension": patch_tensor_info(good, "dim0", 1 << 62, 1),
        "n_dims 0": patch_tensor_info(good, "n_dims", 0, 0),
        "n_dims 5": patch_tensor_info(good, "n_dims", 5, 0),
    }
    for name, blob in cases.items():
        assert status_of(qk, write(tmp_path, blob, "bad.gguf")) == qk.QK_EFORMAT, name


def test_every_truncation_is_rejected(qk, tmp_path):
    """Every proper prefix of a valid file is QK_EFORMAT: the reader checks
    each read against the file size (a prefix that still holds the whole
    index but cuts the data is caught by the tensor bounds)."""
    kvs = KVS[:6] + [KVS[13], KVS[14]]
    ts = [("a", [256, 1], gw.Q4_K, rand_bytes(144, 5)), ("b", [32], gw.F32, rand_bytes(128, 6))]
    blob = gw.build(kvs, ts)
    p = os.path.join(tmp_path, "cut.gguf")
    for n in range(0, len(blob)):
        with open(p, "wb") as fh:
            fh.write(blob[:n])
        assert status_of(qk, p) == qk.QK_EFORMAT, n
    with open(p, "wb") as fh:
        fh.write(blob)
    assert status_of(qk, p) == qk.QK_OK


def test_count_larger_than_file(qk, tmp_path):
    blob = bytearray(gw.build([], []))
    struct.pack_into("<Q", blob, 8, 1 << 40)  # tensor count
    assert status_of(qk, write(tmp_path, bytes(blob), "c.gguf")) == qk.QK_EFORMAT
    blob = bytearray(gw.build([("k", gw.ARRAY, (gw.UINT8, [1, 2]))], []))
    # array count far past the file
    pos = 8 + 16 + 8 + 1 + 4 + 4
    struct.pack_into("<Q", blob, pos, 1 << 50)
    assert status_of(qk, write(tmp_path, bytes(blob), "c.gguf")) == qk.QK_EFORMAT


_BIG_COUNT_CHILD = r"""
import ctypes, resource, sys
resource.setrlimit(resource.RLIMIT_AS, (int(sys.argv[3]), int(sys.argv[3])))
lib = ctypes.CDLL(sys.argv[1])
lib.qk_gguf_open.argtypes = [ctypes.c_char_p, ctypes.POINTER(ctypes.c_void_p)]
h = ctypes.c_void_p()
print(lib.qk_gguf_open(sys.argv[2].encode(), ctypes.byref(h)))
"""


@pytest.mark.parametrize("field,count", [("kv", 1 << 27), ("kv", 1 << 26), ("tensor", 1 << 25), ("tensor", 1 << 24)],
                         ids=["kv-past-bound", "kv-within-bound", "tensor-past-bound", "tensor-within-bound"])
def test_huge_count_in_large_file_is_rejected_without_allocating(qk, tmp_path, field, count):
    """A 1 GiB sparse file whose header claims 2^24..2^27 metadata or tensor
    entries: counts the file cannot hold are rejected before anything is
    read, and counts it could hold fail on the first malformed entry with the
    tables grown only entry by entry. Run in a child process whose address
    space is capped at the file's mapping plus 1.5 GiB, so that sizing the
    tables from the counts (16-112 bytes per claimed entry, 2-15 GB) could
    not pass unnoticed: the call returns QK_EFORMAT instead of aborting."""
    import subprocess
    import sys

    size = 1 << 30
    p = os.path.join(tmp_path, "sparse.gguf")
    with open(p, "wb") as fh:
        fh.write(struct.pack("<IIQQ", 0x46554747, 3, count if field == "tensor" else 0,
                             count if field == "kv" else 0))
        fh.truncate(size)  # the rest reads as zeros (empty keys / names)
    r = subprocess.run([sys.executable, "-c", _BIG_COUNT_CHILD, qk.LIB_PATH, p, str(size + (3 << 29))],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr[-2000:]
    assert int(r.stdout.strip()) == qk.QK_EFORMAT
