"""A test-side GGUF writer, written from the GGUF specification (v2/v3,
little-endian), independent of the library's reader: the suite writes its
own model files, as the picoLM page's runnable file builds a real GGUF file
from scratch and maps it back ("picoLM, in Python", "Run it locally").

Layout: uint32 magic "GGUF", uint32 version, uint64 tensor count, uint64
metadata count; metadata (string key, uint32 type, value); tensor infos
(string name, uint32 n_dims, uint64 dims innermost first, uint32 ggml type,
uint64 offset into the data section); padding to the alignment; the data,
each tensor at a multiple of the alignment. A string is a uint64 length and
its bytes.
"""
from __future__ import annotations

import struct

UINT8, INT8, UINT16, INT16, UINT32, INT32, FLOAT32, BOOL, STRING, ARRAY, UINT64, INT64, FLOAT64 = range(13)
SCALAR_FMT = {UINT8: "B", INT8: "b", UINT16: "H", INT16: "h", UINT32: "I", INT32: "i", FLOAT32: "f", BOOL: "B",
              UINT64: "Q", INT64: "q", FLOAT64: "d"}

# ggml tensor types: (id, weights per block, bytes per block)
F32, F16, Q4_0, Q8_0, Q4_K, Q6_K, Q5_K = (0, 1, 4), (1, 1, 2), (2, 32, 18), (8, 32, 34), (12, 256, 144), \
    (14, 256, 210), (13, 256, 176)


def gstr(s: str | bytes) -> bytes:
    b = s.encode() if isinstance(s, str) else s
    return struct.pack("<Q", len(b)) + b


def value(t: int, v) -> bytes:
    if t == STRING:
        return gstr(v)
    if t == ARRAY:
        et, items = v
        out = struct.pack("<IQ", et, len(items))
        return out + b"".join(value(et, x) for x in items)
    return struct.pack("<" + SCALAR_FMT[t], v)


def tensor_bytes(dims: list[int], gt) -> int:
    n = 1
    for d in dims:
        n *= d
    return n // gt[1] * gt[2]


def build(kvs: list[tuple[str, int, object]], tensors: list[tuple[str, list[int], tuple, bytes]],
          version: int = 3, alignment: int = 32, magic: bytes = b"GGUF") -> bytes:
    """kvs: (key, value type, value); tensors: (name, dims innermost first,
    ggml type tuple, data bytes). `alignment` must match general.alignment
    when kvs set it (32 otherwise)."""
    head = magic + struct.pack("<IQQ", version, len(tensors), len(kvs))
    meta = b"".join(gstr(k) + struct.pack("<I", t) + value(t, v) for k, t, v in kvs)
    infos, rel, off = b"", [], 0
    for name, dims, gt, data in tensors:
        assert len(data) == tensor_bytes(dims, gt), name
        off = (off + alignment - 1) // alignment * alignment
        rel.append(off)
        infos += gstr(name) + struct.pack("<I", len(dims)) + struct.pack("<%dQ" % len(dims), *dims)
        infos += struct.pack("<IQ", gt[0], off)
        off += len(data)
    out = bytearray(head + meta + infos)
    data0 = (len(out) + alignment - 1) // alignment * alignment
    out += b"\0" * (data0 - len(out))
    for (name, dims, gt, data), r in zip(tensors, rel):
        out += b"\0" * (data0 + r - len(out))
        out += data
    return bytes(out)


def data_start(blob: bytes, alignment: int = 32) -> int:
    """Offset of the data section of a file build() wrote, recomputed by
    walking its header (used to check the reader's absolute offsets)."""
    pos = 4 + 4
    nt, nkv = struct.unpack_from("<QQ", blob, pos)
    pos += 16

    def skip_value(t: int, p: int) -> int:
        if t == STRING:
            (n,) = struct.unpack_from("<Q", blob, p)
            return p + 8 + n
        if t == ARRAY:
            et, n = struct.unpack_from("<IQ", blob, p)
            p += 12
            for _ in range(n):
                p = skip_value(et, p)
            return p
        return p + struct.calcsize("<" + SCALAR_FMT[t])

    for _ in range(nkv):
        (n,) = struct.unpack_from("<Q", blob, pos)
        pos += 8 + n
        (t,) = struct.unpack_from("<I", blob, pos)
        pos = skip_value(t, pos + 4)
    for _ in range(nt):
        (n,) = struct.unpack_from("<Q", blob, pos)
        pos += 8 + n
        (nd,) = struct.unpack_from("<I", blob, pos)
        pos += 4 + 8 * nd + 4 + 8
    return (pos + alignment - 1) // alignment * alignment
