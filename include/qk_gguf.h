/*
 * qk_gguf.h — reading a GGUF model file on the host, and uploading its
 * tensors to the GPU for the compute calls of qk.h.
 *
 * What the file holds ("picoLM, in Python", section "§1 — GGUF, and why it
 * is mmap-able"): a header, self-describing key/value metadata, a tensor
 * index of (name, shape, type, offset), padding to general.alignment, then
 * one blob of tensor data; every tensor is a byte range at a known offset,
 * so the file is mapped, not loaded. The byte encoding those pages do not
 * spell out is the GGUF specification's (versions 2 and 3, little-endian):
 *
 *   uint32 magic "GGUF", uint32 version, uint64 tensor count, uint64
 *   metadata count; metadata entries (string key, uint32 value type,
 *   value); tensor infos (string name, uint32 n_dims, uint64 dims[n_dims]
 *   innermost first, uint32 ggml type, uint64 offset into the data
 *   section); the data section starts at the next multiple of the
 *   alignment (metadata "general.alignment", uint32, default 32) and every
 *   offset is a multiple of it. A string is a uint64 length and that many
 *   bytes (no terminator); an array is a uint32 element type, a uint64
 *   count and the elements.
 *
 * A weight matrix of `rows` outputs and `cols` inputs has dims {cols, rows}:
 * its bytes are rows x (cols / block) blocks, row-major, which is the W
 * layout of qk.h.
 *
 * Ownership: qk_gguf_open maps the file read-only and parses it; every
 * pointer a query returns (names, strings, tensor data) points into memory
 * owned by the qk_gguf and stays valid until qk_gguf_close. Nothing here
 * touches the GPU except qk_gguf_upload.
 *
 * Errors: calls return a qk_status (qk.h). A file that is not GGUF v2/v3, is
 * truncated, or whose index is inconsistent (a tensor past the end of the
 * file, an offset that is not a multiple of the alignment, a dimension that
 * is not a whole number of blocks, an unknown tensor type) is QK_EFORMAT:
 * every read is checked against the file size, so no file makes the reader
 * read outside it.
 */
#ifndef QK_GGUF_H
#define QK_GGUF_H

#include <stdint.h>

#include "qk.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct qk_gguf qk_gguf;

/* Metadata value types (GGUF specification numbering). */
typedef enum {
    QK_GGUF_UINT8 = 0,
    QK_GGUF_INT8 = 1,
    QK_GGUF_UINT16 = 2,
    QK_GGUF_INT16 = 3,
    QK_GGUF_UINT32 = 4,
    QK_GGUF_INT32 = 5,
    QK_GGUF_FLOAT32 = 6,
    QK_GGUF_BOOL = 7,
    QK_GGUF_STRING = 8,
    QK_GGUF_ARRAY = 9,
    QK_GGUF_UINT64 = 10,
    QK_GGUF_INT64 = 11,
    QK_GGUF_FLOAT64 = 12
} qk_gguf_value_type;

/* One entry of the tensor index. */
typedef struct qk_gguf_tensor {
    const char *name; /* NUL-terminated */
    int n_dims;       /* 1..4 */
    int64_t dims[4];  /* dims[0] innermost (columns); unused entries 1 */
    int ggml_type;    /* the file's tensor type id (ggml numbering: 0 F32,
                         1 F16, 2 Q4_0, 8 Q8_0 with an fp16 scale, 12 Q4_K,
                         14 Q6_K, ...) */
    int qk_type;      /* the qk_type the compute calls take for these bytes:
                         QK_Q4_0, QK_Q4_K, QK_Q6_K, QK_Q5_K, QK_Q2_K,
                         QK_Q3_K, QK_Q5_1, or QK_Q8_0_F16 for GGUF's Q8_0
                         (not this library's 36-byte QK_Q8_0); 0 for any
                         other type */
    int64_t offset;   /* byte offset of the data from the start of the file */
    int64_t nbytes;   /* bytes of the data */
    const void *data; /* the data in the mapped file (host memory) */
} qk_gguf_tensor;

/* Map and parse `path`. On success *out is a new handle (QK_OK); on failure
 * *out is NULL and the status is QK_EIO (cannot open or map), QK_EFORMAT,
 * QK_ENOMEM (host memory ran out) or QK_EINVAL_PTR (a NULL argument). Entry
 * counts that the file cannot hold are QK_EFORMAT before anything is
 * allocated, and the tables grow as entries are read, so a truncated file
 * fails without allocating much more than its own size. */
int qk_gguf_open(const char *path, qk_gguf **out);

/* Unmap and free; NULL is a no-op. */
void qk_gguf_close(qk_gguf *g);

/* The file's version (2 or 3), its alignment, its tensor and metadata
 * counts; a negative qk_status for a NULL handle. */
int qk_gguf_version(const qk_gguf *g);
int64_t qk_gguf_alignment(const qk_gguf *g);
int64_t qk_gguf_tensor_count(const qk_gguf *g);
int64_t qk_gguf_kv_count(const qk_gguf *g);

/* Tensor i of the index (0 <= i < tensor count), else QK_ENOTFOUND. */
int qk_gguf_tensor_info(const qk_gguf *g, int64_t i, qk_gguf_tensor *out);

/* Index of the tensor or metadata key with this name, or QK_ENOTFOUND. */
int64_t qk_gguf_find_tensor(const qk_gguf *g, const char *name);
int64_t qk_gguf_find_key(const qk_gguf *g, const char *key);

/* Key and value type of metadata entry i. */
int qk_gguf_key(const qk_gguf *g, int64_t i, const char **key, int *value_type);

/* The value of entry i: any integer type or bool as int64 (uint64 above
 * INT64_MAX is QK_EINVAL_TYPE), float32/float64 as double, a string as a
 * NUL-terminated copy and its length. Another value type is QK_EINVAL_TYPE. */
int qk_gguf_get_int(const qk_gguf *g, int64_t i, int64_t *out);
int qk_gguf_get_float(const qk_gguf *g, int64_t i, double *out);
int qk_gguf_get_string(const qk_gguf *g, int64_t i, const char **s, int64_t *len);

/* An array entry: its element type and count, and for fixed-size element
 * types the packed little-endian elements in the mapped file (*data NULL for
 * an array of strings: read those with qk_gguf_get_array_string). */
int qk_gguf_get_array(const qk_gguf *g, int64_t i, int *elem_type, int64_t *count, const void **data);
int qk_gguf_get_array_string(const qk_gguf *g, int64_t i, int64_t j, const char **s, int64_t *len);

/* Copy tensor i's bytes to device memory dst (at least nbytes, owned by the
 * caller) with hipMemcpyAsync on `stream` (a hipStream_t as void*, NULL the
 * null stream). The source is the mapped file, so the copy is staged by the
 * HIP runtime; the call returns once the copy is enqueued and the caller
 * synchronises before using dst. QK_EHIP if the runtime refuses the copy. */
int qk_gguf_upload(const qk_gguf *g, int64_t i, void *dst, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QK_GGUF_H */
