// qk_gguf.cpp — the GGUF reader of include/qk_gguf.h.
//
// The file is mapped read-only and parsed once with a cursor that checks
// every read against the file size; the index and the metadata are kept as
// owned copies (names and strings NUL-terminated), tensor data and packed
// array elements as pointers into the mapping. Layout: a header, key/value
// metadata, the tensor index, padding to general.alignment, one data blob
// ("picoLM, in Python", "§1 — GGUF, and why it is mmap-able"); the byte
// encoding is the GGUF specification's (see the header).
#include <fcntl.h>
#include <hip/hip_runtime_api.h>
#include <sys/mman.h>
#include <sys/stat.h>
#include <unistd.h>

#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/qk_gguf.h"
#include "qk_launch.h"

namespace {

constexpr uint32_t kMagic = 0x46554747u;  // "GGUF" as a little-endian uint32
constexpr int kMaxDims = 4;

// Block size (weights) and block bytes of the ggml tensor types a model file
// may hold; 0 for ids this reader does not know.
struct GgmlType {
    int elems, bytes, qk;
};
GgmlType ggml_type(uint32_t t) {
    switch (t) {
    case 0: return {1, 4, 0};        // F32
    case 1: return {1, 2, 0};        // F16
    case 2: return {32, 18, QK_Q4_0};
    case 3: return {32, 20, 0};      // Q4_1
    case 6: return {32, 22, 0};      // Q5_0
    case 7: return {32, 24, QK_Q5_1};
    case 8: return {32, 34, QK_Q8_0_F16};  // Q8_0 (fp16 scale)
    case 9: return {32, 36, 0};      // Q8_1
    case 10: return {256, 84, QK_Q2_K};
    case 11: return {256, 110, QK_Q3_K};
    case 12: return {256, 144, QK_Q4_K};
    case 13: return {256, 176, QK_Q5_K};
    case 14: return {256, 210, QK_Q6_K};
    case 15: return {256, 292, 0};   // Q8_K
    case 24: return {1, 1, 0};       // I8
    case 25: return {1, 2, 0};       // I16
    case 26: return {1, 4, 0};       // I32
    case 27: return {1, 8, 0};       // I64
    case 28: return {1, 8, 0};       // F64
    case 30: return {1, 2, 0};       // BF16
    default: return {0, 0, 0};
    }
}

// Bytes of one element of a fixed-size metadata value type; 0 for string,
// array or an unknown type.
int64_t scalar_bytes(uint32_t t) {
    switch (t) {
    case QK_GGUF_UINT8: case QK_GGUF_INT8: case QK_GGUF_BOOL: return 1;
    case QK_GGUF_UINT16: case QK_GGUF_INT16: return 2;
    case QK_GGUF_UINT32: case QK_GGUF_INT32: case QK_GGUF_FLOAT32: return 4;
    case QK_GGUF_UINT64: case QK_GGUF_INT64: case QK_GGUF_FLOAT64: return 8;
    default: return 0;
    }
}

struct Cursor {
    const uint8_t *base;
    uint64_t size, pos;
    bool ok = true;

    bool need(uint64_t n) {
        if (!ok || n > size - pos) ok = false;
        return ok;
    }
    template <class T> T get() {
        T v{};
        if (need(sizeof(T))) {
            std::memcpy(&v, base + pos, sizeof(T));
            pos += sizeof(T);
        }
        return v;
    }
    std::string str() {
        const uint64_t n = get<uint64_t>();
        if (!need(n)) return {};
        std::string s(reinterpret_cast<const char *>(base + pos), (size_t)n);
        pos += n;
        return s;
    }
    void skip(uint64_t n) {
        if (need(n)) pos += n;
    }
};

struct Value {
    uint32_t type = 0;
    int64_t i = 0;              // integer types and bool
    uint64_t u = 0;             // uint64 (may exceed int64)
    double f = 0.0;             // float types
    std::string s;              // string
    uint32_t elem = 0;          // array element type
    int64_t count = 0;          // array element count
    const void *data = nullptr; // fixed-size array elements in the mapping
    std::vector<std::string> strs;  // string array elements
};

bool read_scalar(Cursor &c, uint32_t t, Value &v) {
    switch (t) {
    case QK_GGUF_UINT8: v.i = c.get<uint8_t>(); break;
    case QK_GGUF_INT8: v.i = c.get<int8_t>(); break;
    case QK_GGUF_UINT16: v.i = c.get<uint16_t>(); break;
    case QK_GGUF_INT16: v.i = c.get<int16_t>(); break;
    case QK_GGUF_UINT32: v.i = c.get<uint32_t>(); break;
    case QK_GGUF_INT32: v.i = c.get<int32_t>(); break;
    case QK_GGUF_BOOL: {
        const uint8_t b = c.get<uint8_t>();
        if (b > 1) return false;
        v.i = b;
        break;
    }
    case QK_GGUF_UINT64: v.u = c.get<uint64_t>(); v.i = (int64_t)v.u; break;
    case QK_GGUF_INT64: v.i = c.get<int64_t>(); break;
    case QK_GGUF_FLOAT32: v.f = c.get<float>(); break;
    case QK_GGUF_FLOAT64: v.f = c.get<double>(); break;
    case QK_GGUF_STRING: v.s = c.str(); break;
    default: return false;
    }
    return c.ok;
}

bool read_value(Cursor &c, uint32_t t, Value &v) {
    v.type = t;
    if (t != QK_GGUF_ARRAY) return read_scalar(c, t, v);
    v.elem = c.get<uint32_t>();
    const uint64_t n = c.get<uint64_t>();
    if (!c.ok || n > (uint64_t)INT64_MAX) return false;
    v.count = (int64_t)n;
    if (v.elem == QK_GGUF_STRING) {
        // each element takes at least its 8-byte length; the list grows as
        // elements are read
        if (n > (c.size - c.pos) / 8) return false;
        for (uint64_t j = 0; j < n && c.ok; j++) v.strs.push_back(c.str());
        return c.ok;
    }
    const int64_t eb = scalar_bytes(v.elem);
    if (eb == 0) return false;  // arrays of arrays are not used by model files
    if (n > (c.size - c.pos) / (uint64_t)eb) return false;
    v.data = c.base + c.pos;
    c.skip(n * (uint64_t)eb);
    return c.ok;
}

}  // namespace

struct qk_gguf {
    void *map = nullptr;
    uint64_t size = 0;
    int version = 0;
    int64_t alignment = 32;
    std::vector<std::string> keys;
    std::vector<Value> values;
    std::unordered_map<std::string, int64_t> key_index, tensor_index;
    std::vector<std::string> names;
    std::vector<qk_gguf_tensor> tensors;
};

namespace {

int fmt(const char *msg) { return qk::set_last_error(QK_EFORMAT, msg); }

int parse(qk_gguf *g) {
    Cursor c{static_cast<const uint8_t *>(g->map), g->size, 0};
    if (c.get<uint32_t>() != kMagic || !c.ok) return fmt("no GGUF magic");
    const uint32_t version = c.get<uint32_t>();
    if (!c.ok || (version != 2 && version != 3)) return fmt("unsupported GGUF version (2 and 3 are read)");
    g->version = (int)version;
    const uint64_t nt = c.get<uint64_t>(), nkv = c.get<uint64_t>();
    if (!c.ok) return fmt("truncated header");
    // A metadata entry takes at least 13 bytes (key length, value type, a
    // one-byte value) and a tensor entry at least 32 (name length, dimension
    // count, one dimension, type, offset): counts that the rest of the file
    // cannot hold are rejected before anything is read, and the tables grow
    // entry by entry, so a truncated file fails before much is allocated.
    const uint64_t rest = c.size - c.pos;
    if (nkv > rest / 13 || nt > rest / 32 || nkv * 13 > rest - nt * 32)
        return fmt("tensor or metadata count larger than the file");
    for (uint64_t i = 0; i < nkv; i++) {
        std::string key = c.str();
        const uint32_t t = c.get<uint32_t>();
        Value v;
        if (!c.ok || !read_value(c, t, v)) return fmt("truncated or malformed metadata entry");
        if (!g->key_index.emplace(key, (int64_t)i).second) return fmt("duplicate metadata key");
        g->values.push_back(v);
        g->keys.push_back(std::move(key));
    }
    auto al = g->key_index.find("general.alignment");
    if (al != g->key_index.end()) {
        const Value &v = g->values[al->second];
        if (v.type != QK_GGUF_UINT32 || v.i <= 0 || (v.i & (v.i - 1)) != 0)
            return fmt("general.alignment is not a power of two uint32");
        g->alignment = v.i;
    }
    std::vector<uint64_t> rel;
    for (uint64_t i = 0; i < nt; i++) {
        std::string name = c.str();
        const uint32_t nd = c.get<uint32_t>();
        if (!c.ok || nd < 1 || nd > kMaxDims) return fmt("truncated tensor info or bad dimension count");
        g->tensors.push_back(qk_gguf_tensor{});
        rel.push_back(0);
        qk_gguf_tensor &t = g->tensors.back();
        t.n_dims = (int)nd;
        uint64_t elems = 1;
        for (int d = 0; d < kMaxDims; d++) {
            uint64_t v = 1;
            if (d < (int)nd) v = c.get<uint64_t>();
            if (!c.ok || v == 0 || v > ((uint64_t)1 << 40)) return fmt("bad tensor dimension");
            if (elems > UINT64_MAX / v) return fmt("tensor size overflows");
            elems *= v;
            t.dims[d] = (int64_t)v;
        }
        const uint32_t type = c.get<uint32_t>();
        rel[i] = c.get<uint64_t>();
        if (!c.ok) return fmt("truncated tensor info");
        const GgmlType gt = ggml_type(type);
        if (gt.elems == 0) return fmt("unknown tensor type");
        if (t.dims[0] % gt.elems != 0) return fmt("innermost dimension is not a whole number of blocks");
        const uint64_t blocks = elems / (uint64_t)gt.elems;
        if (blocks > (uint64_t)INT64_MAX / (uint64_t)gt.bytes) return fmt("tensor size overflows");
        t.nbytes = (int64_t)(blocks * (uint64_t)gt.bytes);
        t.ggml_type = (int)type;
        t.qk_type = gt.qk;
        if (rel[i] % (uint64_t)g->alignment != 0) return fmt("tensor offset is not a multiple of the alignment");
        if (!g->tensor_index.emplace(name, (int64_t)i).second) return fmt("duplicate tensor name");
        g->names.push_back(std::move(name));
    }
    const uint64_t a = (uint64_t)g->alignment;
    const uint64_t data0 = (c.pos + a - 1) / a * a;
    if (data0 > g->size && nt > 0) return fmt("data section starts past the end of the file");
    for (uint64_t i = 0; i < nt; i++) {
        qk_gguf_tensor &t = g->tensors[i];
        if (rel[i] > g->size || data0 > g->size - rel[i] || (uint64_t)t.nbytes > g->size - data0 - rel[i])
            return fmt("tensor data past the end of the file");
        t.offset = (int64_t)(data0 + rel[i]);
        t.data = static_cast<const uint8_t *>(g->map) + t.offset;
        t.name = g->names[i].c_str();
    }
    return QK_OK;
}

bool valid(const qk_gguf *g) { return g != nullptr; }

}  // namespace

extern "C" {

int qk_gguf_open(const char *path, qk_gguf **out) {
    if (!out) return qk::set_last_error(QK_EINVAL_PTR, "out is NULL");
    *out = nullptr;
    if (!path) return qk::set_last_error(QK_EINVAL_PTR, "path is NULL");
    const int fd = open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return qk::set_last_error(QK_EIO, "cannot open the file");
    struct stat st;
    if (fstat(fd, &st) != 0) {
        close(fd);
        return qk::set_last_error(QK_EIO, "cannot stat the file");
    }
    if (st.st_size <= 0) {
        close(fd);
        return qk::set_last_error(QK_EFORMAT, "empty file");
    }
    void *m = mmap(nullptr, (size_t)st.st_size, PROT_READ, MAP_PRIVATE, fd, 0);
    close(fd);
    if (m == MAP_FAILED) return qk::set_last_error(QK_EIO, "cannot map the file");
    qk_gguf *g = new (std::nothrow) qk_gguf;
    if (!g) {
        munmap(m, (size_t)st.st_size);
        return qk::set_last_error(QK_ENOMEM, "out of host memory");
    }
    g->map = m;
    g->size = (uint64_t)st.st_size;
    int s;
    try {
        s = parse(g);
    } catch (const std::bad_alloc &) {
        s = qk::set_last_error(QK_ENOMEM, "out of host memory while reading the file's tables");
    }
    if (s != QK_OK) {
        qk_gguf_close(g);
        return s;
    }
    *out = g;
    qk::set_last_error(QK_OK, "");
    return QK_OK;
}

void qk_gguf_close(qk_gguf *g) {
    if (!g) return;
    if (g->map) munmap(g->map, (size_t)g->size);
    delete g;
}

int qk_gguf_version(const qk_gguf *g) { return valid(g) ? g->version : QK_EINVAL_PTR; }
int64_t qk_gguf_alignment(const qk_gguf *g) { return valid(g) ? g->alignment : QK_EINVAL_PTR; }
int64_t qk_gguf_tensor_count(const qk_gguf *g) { return valid(g) ? (int64_t)g->tensors.size() : QK_EINVAL_PTR; }
int64_t qk_gguf_kv_count(const qk_gguf *g) { return valid(g) ? (int64_t)g->values.size() : QK_EINVAL_PTR; }

int qk_gguf_tensor_info(const qk_gguf *g, int64_t i, qk_gguf_tensor *out) {
    if (!valid(g) || !out) return QK_EINVAL_PTR;
    if (i < 0 || i >= (int64_t)g->tensors.size()) return QK_ENOTFOUND;
    *out = g->tensors[(size_t)i];
    return QK_OK;
}

int64_t qk_gguf_find_tensor(const qk_gguf *g, const char *name) {
    if (!valid(g) || !name) return QK_EINVAL_PTR;
    auto it = g->tensor_index.find(name);
    return it == g->tensor_index.end() ? QK_ENOTFOUND : it->second;
}

int64_t qk_gguf_find_key(const qk_gguf *g, const char *key) {
    if (!valid(g) || !key) return QK_EINVAL_PTR;
    auto it = g->key_index.find(key);
    return it == g->key_index.end() ? QK_ENOTFOUND : it->second;
}

static const Value *value_at(const qk_gguf *g, int64_t i) {
    if (!valid(g) || i < 0 || i >= (int64_t)g->values.size()) return nullptr;
    return &g->values[(size_t)i];
}

int qk_gguf_key(const qk_gguf *g, int64_t i, const char **key, int *value_type) {
    if (!valid(g)) return QK_EINVAL_PTR;
    const Value *v = value_at(g, i);
    if (!v) return QK_ENOTFOUND;
    if (key) *key = g->keys[(size_t)i].c_str();
    if (value_type) *value_type = (int)v->type;
    return QK_OK;
}

int qk_gguf_get_int(const qk_gguf *g, int64_t i, int64_t *out) {
    if (!valid(g) || !out) return QK_EINVAL_PTR;
    const Value *v = value_at(g, i);
    if (!v) return QK_ENOTFOUND;
    switch (v->type) {
    case QK_GGUF_UINT8: case QK_GGUF_INT8: case QK_GGUF_UINT16: case QK_GGUF_INT16: case QK_GGUF_UINT32:
    case QK_GGUF_INT32: case QK_GGUF_BOOL: case QK_GGUF_INT64:
        *out = v->i;
        return QK_OK;
    case QK_GGUF_UINT64:
        if (v->u > (uint64_t)INT64_MAX) return QK_EINVAL_TYPE;
        *out = (int64_t)v->u;
        return QK_OK;
    default: return QK_EINVAL_TYPE;
    }
}

int qk_gguf_get_float(const qk_gguf *g, int64_t i, double *out) {
    if (!valid(g) || !out) return QK_EINVAL_PTR;
    const Value *v = value_at(g, i);
    if (!v) return QK_ENOTFOUND;
    if (v->type != QK_GGUF_FLOAT32 && v->type != QK_GGUF_FLOAT64) return QK_EINVAL_TYPE;
    *out = v->f;
    return QK_OK;
}

int qk_gguf_get_string(const qk_gguf *g, int64_t i, const char **s, int64_t *len) {
    if (!valid(g) || !s) return QK_EINVAL_PTR;
    const Value *v = value_at(g, i);
    if (!v) return QK_ENOTFOUND;
    if (v->type != QK_GGUF_STRING) return QK_EINVAL_TYPE;
    *s = v->s.c_str();
    if (len) *len = (int64_t)v->s.size();
    return QK_OK;
}

int qk_gguf_get_array(const qk_gguf *g, int64_t i, int *elem_type, int64_t *count, const void **data) {
    if (!valid(g)) return QK_EINVAL_PTR;
    const Value *v = value_at(g, i);
    if (!v) return QK_ENOTFOUND;
    if (v->type != QK_GGUF_ARRAY) return QK_EINVAL_TYPE;
    if (elem_type) *elem_type = (int)v->elem;
    if (count) *count = v->count;
    if (data) *data = v->data;
    return QK_OK;
}

int qk_gguf_get_array_string(const qk_gguf *g, int64_t i, int64_t j, const char **s, int64_t *len) {
    if (!valid(g) || !s) return QK_EINVAL_PTR;
    const Value *v = value_at(g, i);
    if (!v) return QK_ENOTFOUND;
    if (v->type != QK_GGUF_ARRAY || v->elem != QK_GGUF_STRING) return QK_EINVAL_TYPE;
    if (j < 0 || j >= (int64_t)v->strs.size()) return QK_ENOTFOUND;
    *s = v->strs[(size_t)j].c_str();
    if (len) *len = (int64_t)v->strs[(size_t)j].size();
    return QK_OK;
}

int qk_gguf_upload(const qk_gguf *g, int64_t i, void *dst, void *stream) {
    if (!valid(g) || !dst) return qk::set_last_error(QK_EINVAL_PTR, "handle or dst is NULL");
    if (i < 0 || i >= (int64_t)g->tensors.size()) return qk::set_last_error(QK_ENOTFOUND, "no such tensor");
    const qk_gguf_tensor &t = g->tensors[(size_t)i];
    const hipError_t e =
        hipMemcpyAsync(dst, t.data, (size_t)t.nbytes, hipMemcpyHostToDevice, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) {
        char msg[256];
        snprintf(msg, sizeof msg, "hipMemcpyAsync: %s (%d)", hipGetErrorString(e), (int)e);
        return qk::set_last_error(QK_EHIP, msg);
    }
    return QK_OK;
}

}  // extern "C"
