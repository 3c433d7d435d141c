// qk_api.hip — the C ABI of include/qk.h: argument checks, the format
// dispatch table and launch error reporting.
//
// Every check runs on the host before any HIP call; a failed check returns
// its status without launching anything. Formats dispatch through one table
// (block size, block bytes) and a switch in each launcher; every format has a
// fused GEMV — there is no dequantise-then-dot fallback on the GEMV path
// (picoLM fuses only Q4_K and Q6_K and sends the rest through a dequantise-
// then-dot branch, "PicoLM Q6_K量化Bug调试全记录", 方法论; PETIT picks its
// kernel from the header's quant field, "How the pieces match").
#include <atomic>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <set>
#include <tuple>
#include <utility>
#include <vector>

#include "../../include/qk.h"
#include "../../include/qk_step.h"
#include "qk_launch.h"

namespace {

struct FormatInfo {
    int elems;
    int bytes;
};

// Indexed by format id (0 is unused).
constexpr FormatInfo kFormats[] = {{0, 0},    {32, 18},   {32, 36},  {256, 144}, {256, 210},
                                   {32, 34},  {32, 24},   {256, 176}, {256, 84}, {256, 110}};
constexpr int kNumFormats = sizeof(kFormats) / sizeof(kFormats[0]);
static_assert(kNumFormats == QK_Q3_K + 1, "format table covers every id");

thread_local char g_err[512];

int fail(int status, const char *msg) {
    snprintf(g_err, sizeof g_err, "%s", msg);
    return status;
}

const FormatInfo *format_of(int type) {
    if (type <= 0 || type >= kNumFormats) return nullptr;
    return &kFormats[type];
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return na && nb && a0 < b0 + nb && b0 < a0 + na;
}

int hip_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return QK_OK;
    snprintf(g_err, sizeof g_err, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
    return QK_EHIP;
}

// Validates a weight matrix description; on success sets *row_bytes.
int check_matrix(int type, const void *W, int64_t rows, int64_t cols, int64_t *row_bytes) {
    const FormatInfo *f = format_of(type);
    if (!f) return fail(QK_EINVAL_TYPE, "unknown format id");
    if (rows < 0 || cols < 0) return fail(QK_EINVAL_SHAPE, "negative size");
    if (cols % f->elems != 0) return fail(QK_EINVAL_SHAPE, "cols is not a whole number of blocks (pad rows to the block size)");
    const int64_t rb = cols / f->elems * f->bytes;
    if (rows > 0 && rb > 0 && rows > INT64_MAX / rb) return fail(QK_EINVAL_SHAPE, "matrix size overflows");
    if (cols > ((int64_t)1 << 40)) return fail(QK_EINVAL_SHAPE, "cols too large");
    *row_bytes = rb;
    return QK_OK;
}

// Pointer checks for a matrix that will be read (rows > 0, cols > 0).
int check_weights_ptr(const void *W) {
    if (!W) return fail(QK_EINVAL_PTR, "W is NULL");
    if (!aligned(W, 16)) return fail(QK_EALIGN, "W must be 16-byte aligned");
    return QK_OK;
}

}  // namespace

namespace qk {

int device_cu_count() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    {
        std::lock_guard<std::mutex> lk(mu);
        if (cache[dev] > 0) return cache[dev];
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    std::lock_guard<std::mutex> lk(mu);
    cache[dev] = n;
    return n;
}

int device_lds_per_block() {
    static std::mutex mu;
    static int cache[64] = {0};
    int dev = 0;
    // without a device (host-side queries): gfx950's 160 KiB
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 163840;
    {
        std::lock_guard<std::mutex> lk(mu);
        if (cache[dev] > 0) return cache[dev];
    }
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || n <= 0) n = 163840;
    std::lock_guard<std::mutex> lk(mu);
    cache[dev] = n;
    return n;
}

hipError_t allow_max_dynamic_lds(const void *kern) {
    static std::mutex mu;
    static std::set<std::pair<int, const void *>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const int limit = device_lds_per_block();
    std::lock_guard<std::mutex> lk(mu);
    if (done.count({dev, kern})) return hipSuccess;
    hipFuncAttributes fa;
    e = hipFuncGetAttributes(&fa, kern);
    if (e == hipSuccess)
        e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, limit - (int)fa.sharedSizeBytes);
    if (e == hipSuccess) done.insert({dev, kern});
    return e;
}

int occupancy(const void *kern, int threads, size_t lds_bytes) {
    static std::mutex mu;
    static std::map<std::tuple<int, const void *, int, size_t>, int> cache;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = -1;
    const auto key = std::make_tuple(dev, kern, threads, lds_bytes);
    {
        std::lock_guard<std::mutex> lk(mu);
        auto it = cache.find(key);
        if (it != cache.end()) return it->second;
    }
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, lds_bytes) != hipSuccess || nb <= 0) nb = 1;
    std::lock_guard<std::mutex> lk(mu);
    cache[key] = nb;
    return nb;
}

// Tuning overrides (qk_set_tuning): -1 is the table's own choice.
static std::atomic<int> g_tune[QK_TUNE_COUNT] = {-1, -1, -1, -1, -1, -1, -1, -1, -1, -1};
static_assert(QK_TUNE_COUNT == 10, "one initialiser per tuning key");

int tuning(int key) { return key >= 0 && key < QK_TUNE_COUNT ? g_tune[key].load(std::memory_order_relaxed) : -1; }

}  // namespace qk

int qk::set_last_error(int status, const char *msg) { return fail(status, msg); }

namespace qk {
// The kernel a GEMM runs (qk_gemm.hip): a qk_gemm_path value.
int gemm_path(int type, int64_t rows, int64_t cols, int64_t M);
}  // namespace qk

extern "C" {

int qk_block_elems(int type) {
    const FormatInfo *f = format_of(type);
    return f ? f->elems : QK_EINVAL_TYPE;
}

int qk_block_bytes(int type) {
    const FormatInfo *f = format_of(type);
    return f ? f->bytes : QK_EINVAL_TYPE;
}

int64_t qk_row_bytes(int type, int64_t cols) {
    const FormatInfo *f = format_of(type);
    if (!f) return QK_EINVAL_TYPE;
    if (cols < 0 || cols % f->elems != 0) return QK_EINVAL_SHAPE;
    return cols / f->elems * f->bytes;
}

const char *qk_strerror(int status) {
    switch (status) {
    case QK_OK: return "ok";
    case QK_EINVAL_TYPE: return "unknown block format";
    case QK_EINVAL_SHAPE: return "invalid shape";
    case QK_EINVAL_PTR: return "null pointer";
    case QK_EALIGN: return "misaligned pointer";
    case QK_EHIP: return "HIP runtime error";
    case QK_EIO: return "cannot open or map the file";
    case QK_EFORMAT: return "not a well-formed GGUF file";
    case QK_ENOTFOUND: return "no such tensor or key";
    case QK_ENOMEM: return "out of host memory";
    default: return "unknown status";
    }
}

const char *qk_last_error(void) { return g_err; }

const char *qk_last_hip_error(void) { return g_err; }

int qk_set_tuning(int key, int value) {
    if (key < 0 || key >= QK_TUNE_COUNT) return fail(QK_EINVAL_SHAPE, "unknown tuning key");
    if (value < -1) return fail(QK_EINVAL_SHAPE, "tuning value below -1");
    return qk::g_tune[key].exchange(value, std::memory_order_relaxed);
}

int qk_get_tuning(int key) {
    if (key < 0 || key >= QK_TUNE_COUNT) return fail(QK_EINVAL_SHAPE, "unknown tuning key");
    return qk::g_tune[key].load(std::memory_order_relaxed);
}

int qk_dequantize_row_async(int type, const void *blocks, int64_t n, float *out, void *stream) {
    g_err[0] = 0;
    const FormatInfo *f = format_of(type);
    if (!f) return fail(QK_EINVAL_TYPE, "unknown format id");
    if (n < 0 || n % f->elems != 0) return fail(QK_EINVAL_SHAPE, "n is negative or not a whole number of blocks");
    if (n == 0) return QK_OK;
    if (!blocks || !out) return fail(QK_EINVAL_PTR, "blocks or out is NULL");
    if (!aligned(blocks, 16)) return fail(QK_EALIGN, "blocks must be 16-byte aligned");
    if (!aligned(out, 4)) return fail(QK_EALIGN, "out must be 4-byte aligned");
    return hip_status(qk::launch_dequant(type, blocks, n, out, (hipStream_t)stream), "dequantize launch");
}

int qk_dequantize_row(int type, const void *blocks, int64_t n, float *out) {
    return qk_dequantize_row_async(type, blocks, n, out, nullptr);
}

int qk_gemv(int type, const void *W, int64_t rows, int64_t cols, const float *x, float *y, void *stream) {
    g_err[0] = 0;
    int64_t rb = 0;
    const int st = check_matrix(type, W, rows, cols, &rb);
    if (st != QK_OK) return st;
    if (rows == 0) return QK_OK;
    if (!y) return fail(QK_EINVAL_PTR, "y is NULL");
    if (!aligned(y, 4)) return fail(QK_EALIGN, "y must be 4-byte aligned");
    if (cols == 0) return hip_status(qk::launch_fill_zero(y, rows, (hipStream_t)stream), "gemv launch");
    if (check_weights_ptr(W) != QK_OK) return check_weights_ptr(W);
    if (!x) return fail(QK_EINVAL_PTR, "x is NULL");
    if (!aligned(x, 16)) return fail(QK_EALIGN, "x must be 16-byte aligned");
    // every workgroup stages all of x when it starts, so a y written over x
    // (or over W) would be read back by workgroups that start later
    const size_t ny = (size_t)rows * sizeof(float);
    if (overlaps(y, ny, W, (size_t)(rows * rb)) || overlaps(y, ny, x, (size_t)cols * sizeof(float)))
        return fail(QK_EINVAL_PTR, "y overlaps W or x");
    return hip_status(qk::launch_gemv(type, W, rows, cols, x, y, (hipStream_t)stream), "gemv launch");
}

namespace {

// Checks one descriptor as qk_gemv would.
int check_desc(const qk_gemv_desc &d) {
    int64_t rb = 0;
    const int st = check_matrix(d.type, d.W, d.rows, d.cols, &rb);
    if (st != QK_OK) return st;
    if (d.rows == 0) return QK_OK;
    if (!d.y) return fail(QK_EINVAL_PTR, "y is NULL");
    if (!aligned(d.y, 4)) return fail(QK_EALIGN, "y must be 4-byte aligned");
    if (d.cols == 0) return QK_OK;
    if (check_weights_ptr(d.W) != QK_OK) return check_weights_ptr(d.W);
    if (!d.x) return fail(QK_EINVAL_PTR, "x is NULL");
    if (!aligned(d.x, 16)) return fail(QK_EALIGN, "x must be 16-byte aligned");
    return QK_OK;
}

}  // namespace

int qk_gemv_batch(const qk_gemv_desc *descs, int n, void *stream) {
    g_err[0] = 0;
    if (n < 0) return fail(QK_EINVAL_SHAPE, "negative batch size");
    if (n == 0) return QK_OK;
    if (!descs) return fail(QK_EINVAL_PTR, "descs is NULL");
    for (int i = 0; i < n; i++) {
        const int st = check_desc(descs[i]);
        if (st != QK_OK) return st;
    }
    // outputs may not overlap each other or any input of the batch
    for (int i = 0; i < n; i++) {
        const qk_gemv_desc &a = descs[i];
        const size_t ny = (size_t)a.rows * sizeof(float);
        for (int j = 0; j < n; j++) {
            const qk_gemv_desc &b = descs[j];
            const size_t wb = b.rows > 0 && b.cols > 0 ? (size_t)(b.rows * qk_row_bytes(b.type, b.cols)) : 0;
            const size_t xb = b.rows > 0 ? (size_t)b.cols * sizeof(float) : 0;
            if ((j != i && overlaps(a.y, ny, b.y, (size_t)b.rows * sizeof(float))) || overlaps(a.y, ny, b.W, wb) ||
                overlaps(a.y, ny, b.x, xb))
                return fail(QK_EINVAL_PTR, "an output overlaps another output or an input of the batch");
        }
    }
    hipStream_t s = (hipStream_t)stream;
    bool done[64];
    const int nd = n;
    for (int base = 0; base < nd; base += 64) {
        const int cnt = nd - base < 64 ? nd - base : 64;
        for (int i = 0; i < cnt; i++) done[i] = false;
        for (int i = 0; i < cnt; i++) {
            if (done[i]) continue;
            const qk_gemv_desc &d = descs[base + i];
            done[i] = true;
            if (d.rows == 0) continue;
            if (d.cols == 0) {
                const int st = hip_status(qk::launch_fill_zero(d.y, d.rows, s), "gemv batch launch");
                if (st != QK_OK) return st;
                continue;
            }
            if (!qk::gemv_fusable(d.type, d.rows, d.cols)) {
                const int st = hip_status(qk::launch_gemv(d.type, d.W, d.rows, d.cols, d.x, d.y, s), "gemv batch launch");
                if (st != QK_OK) return st;
                continue;
            }
            // gather following descriptors of the same width and x whose
            // formats can share the launch
            qk::GemvItem items[qk::kGemvMaxMats];
            int k = 0;
            items[k++] = qk::GemvItem{d.type, d.W, d.rows, d.y};
            for (int j = i + 1; j < cnt && k < qk::kGemvMaxMats; j++) {
                const qk_gemv_desc &e = descs[base + j];
                if (!done[j] && e.rows > 0 && e.cols == d.cols && e.x == d.x && qk::gemv_groupable(e.type, d.type) &&
                    qk::gemv_fusable(e.type, e.rows, e.cols)) {
                    items[k++] = qk::GemvItem{e.type, e.W, e.rows, e.y};
                    done[j] = true;
                }
            }
            const int st = hip_status(qk::launch_gemv_group(items, k, d.cols, d.x, s), "gemv batch launch");
            if (st != QK_OK) return st;
        }
    }
    return QK_OK;
}

// ---- the persistent decode pass

struct qk_gemv_pass {
    void *ws;
    int nstages;
    int grid;
    int device;
    int64_t spin_limit;
};

// What a pass's arguments describe, checked: the stages, each stage's input
// (where x and aux come from) and which outputs a later stage reads.
struct PassPlan {
    std::vector<int> first;  // stage s is descs[first[s] .. first[s + 1])
    std::vector<int64_t> cols;
    std::vector<qk::PassStageIn> in;
    std::vector<qk::GemvItem> items;
    std::vector<unsigned char> chained;  // a later stage reads the GEMV's output
    std::vector<int64_t> chained_rows;
};

static int pass_plan(const char *fn, const qk_gemv_desc *descs, int n, const int *stage,
                     const qk_gemv_pass_input *inputs, PassPlan &pp) {
    char msg[192];
    auto bad = [&](int status, const char *what) {
        snprintf(msg, sizeof msg, "%s: %s", fn, what);
        return fail(status, msg);
    };
    if (n < 1) return bad(QK_EINVAL_SHAPE, "no GEMVs");
    if (!descs || !stage) return bad(QK_EINVAL_PTR, "descs or stage is NULL");
    if (stage[0] != 0) return bad(QK_EINVAL_SHAPE, "stage[0] must be 0");
    pp.first.assign(1, 0);
    for (int i = 1; i < n; i++) {
        if (stage[i] != stage[i - 1] && stage[i] != stage[i - 1] + 1)
            return bad(QK_EINVAL_SHAPE, "stage numbers must start at 0 and rise by 0 or 1");
        if (stage[i] != stage[i - 1]) pp.first.push_back(i);
    }
    pp.first.push_back(n);
    const int S = (int)pp.first.size() - 1;
    pp.cols.assign((size_t)S, 0);
    pp.in.assign((size_t)S, qk::PassStageIn{});
    pp.items.assign((size_t)n, qk::GemvItem{});
    pp.chained.assign((size_t)n, 0);
    pp.chained_rows.clear();
    for (int s = 0; s < S; s++) {
        if (pp.first[s + 1] - pp.first[s] > qk::kGemvMaxMats) return bad(QK_EINVAL_SHAPE, "more than 4 GEMVs in a stage");
        const qk_gemv_desc &d0 = descs[pp.first[s]];
        for (int i = pp.first[s]; i < pp.first[s + 1]; i++) {
            const qk_gemv_desc &d = descs[i];
            const int st = check_desc(d);
            if (st != QK_OK) return st;
            if (d.rows < 1 || d.cols != d0.cols || d.x != d0.x)
                return bad(QK_EINVAL_SHAPE, "the GEMVs of a stage need rows, one width and one x");
            if (!qk::pass_stage_ok(d.type, d.rows, d.cols))
                return bad(QK_EINVAL_SHAPE, "a pass takes Q4_K and Q6_K matrices of 256 to 6144 columns that the "
                                            "fused GEMV takes (use qk_gemv_batch for others)");
            pp.items[(size_t)i] = qk::GemvItem{d.type, d.W, d.rows, d.y};
        }
        pp.cols[(size_t)s] = d0.cols;
    }
    // outputs may not overlap a weight matrix or another output
    for (int i = 0; i < n; i++) {
        const qk_gemv_desc &a = descs[i];
        const size_t ny = (size_t)a.rows * sizeof(float);
        for (int j = 0; j < n; j++) {
            const qk_gemv_desc &b = descs[j];
            if ((j != i && overlaps(a.y, ny, b.y, (size_t)b.rows * sizeof(float))) ||
                overlaps(a.y, ny, b.W, (size_t)(b.rows * qk_row_bytes(b.type, b.cols))))
                return bad(QK_EINVAL_PTR, "an output overlaps another output or a weight matrix");
        }
    }
    // An input of stage s is either exactly the output of a GEMV of an
    // earlier stage (whose rows are the stage's width), or overlaps no
    // output at all: -1 then. -2: neither.
    auto source = [&](int s, const float *p, size_t bytes) {
        for (int i = 0; i < n; i++) {
            const qk_gemv_desc &d = descs[i];
            if (!overlaps(p, bytes, d.y, (size_t)d.rows * sizeof(float))) continue;
            return (p == d.y && stage[i] < s && d.rows == pp.cols[(size_t)s]) ? i : -2;
        }
        return -1;
    };
    for (int s = 0; s < S; s++) {
        const int64_t cols = pp.cols[(size_t)s];
        const size_t xb = (size_t)cols * sizeof(float);
        qk::PassStageIn &pi = pp.in[(size_t)s];
        const qk_gemv_pass_input in = inputs ? inputs[s] : qk_gemv_pass_input{QK_PASS_IN_PLAIN, nullptr, nullptr, 0.f};
        if (in.kind != QK_PASS_IN_PLAIN && in.kind != QK_PASS_IN_RMSNORM && in.kind != QK_PASS_IN_SWIGLU)
            return bad(QK_EINVAL_SHAPE, "unknown input kind");
        pi.kind = in.kind;
        pi.x = descs[pp.first[s]].x;
        pi.x_src = source(s, pi.x, xb);
        if (pi.x_src == -2)
            return bad(QK_EINVAL_PTR, "an x overlaps an output without being an earlier stage's whole output");
        if (in.kind == QK_PASS_IN_SWIGLU) {
            if (!in.aux) return bad(QK_EINVAL_PTR, "SwiGLU input without aux");
            if (!aligned(in.aux, 16)) return fail(QK_EALIGN, "qk_gemv_pass: aux must be 16-byte aligned");
            pi.aux = in.aux;
            pi.aux_src = source(s, in.aux, xb);
            if (pi.aux_src == -2)
                return bad(QK_EINVAL_PTR, "an aux overlaps an output without being an earlier stage's whole output");
        } else {
            pi.aux_src = -1;
        }
        if (in.kind == QK_PASS_IN_RMSNORM) {
            if (!(in.eps > 0.f) || !(in.eps < 1e30f)) return bad(QK_EINVAL_SHAPE, "RMSNorm eps must be positive");
            pi.eps = in.eps;
            if (in.norm_w) {
                if (!aligned(in.norm_w, 16)) return fail(QK_EALIGN, "qk_gemv_pass: norm_w must be 16-byte aligned");
                if (source(s, in.norm_w, xb) != -1) return bad(QK_EINVAL_PTR, "norm_w overlaps an output");
                pi.norm_w = in.norm_w;
            }
        }
        if (pi.x_src >= 0) pp.chained[(size_t)pi.x_src] = 1;
        if (pi.aux_src >= 0) pp.chained[(size_t)pi.aux_src] = 1;
    }
    for (int i = 0; i < n; i++)
        if (pp.chained[(size_t)i]) pp.chained_rows.push_back(descs[i].rows);
    return QK_OK;
}

int64_t qk_gemv_pass_workspace_bytes(const qk_gemv_desc *descs, int n, const int *stage,
                                     const qk_gemv_pass_input *inputs) {
    g_err[0] = 0;
    PassPlan pp;
    const int st = pass_plan("qk_gemv_pass_workspace_bytes", descs, n, stage, inputs, pp);
    if (st != QK_OK) return st;
    return qk::pass_workspace_bytes((int)pp.cols.size(), pp.chained_rows.data(), (int)pp.chained_rows.size());
}

int qk_gemv_pass_create(const qk_gemv_desc *descs, int n, const int *stage, const qk_gemv_pass_input *inputs,
                        void *workspace, int64_t workspace_bytes, qk_gemv_pass **out) {
    g_err[0] = 0;
    if (!out) return fail(QK_EINVAL_PTR, "qk_gemv_pass_create: out is NULL");
    *out = nullptr;
    PassPlan pp;
    const int st = pass_plan("qk_gemv_pass_create", descs, n, stage, inputs, pp);
    if (st != QK_OK) return st;
    const int S = (int)pp.cols.size();
    if (!workspace) return fail(QK_EINVAL_PTR, "qk_gemv_pass_create: workspace is NULL");
    if (!aligned(workspace, 256)) return fail(QK_EALIGN, "qk_gemv_pass_create: workspace must be 256-byte aligned");
    if (workspace_bytes < qk::pass_workspace_bytes(S, pp.chained_rows.data(), (int)pp.chained_rows.size()))
        return fail(QK_EINVAL_SHAPE, "qk_gemv_pass_create: workspace smaller than qk_gemv_pass_workspace_bytes()");
    // the workspace may not overlap a weight matrix, an input or an output
    for (int i = 0; i < n; i++) {
        const qk_gemv_desc &d = descs[i];
        if (overlaps(workspace, (size_t)workspace_bytes, d.W, (size_t)(d.rows * qk_row_bytes(d.type, d.cols))) ||
            overlaps(workspace, (size_t)workspace_bytes, d.y, (size_t)d.rows * sizeof(float)) ||
            overlaps(workspace, (size_t)workspace_bytes, d.x, (size_t)d.cols * sizeof(float)))
            return fail(QK_EINVAL_PTR, "qk_gemv_pass_create: the workspace overlaps a matrix, an input or an output");
    }
    for (size_t s = 0; s < pp.in.size(); s++) {
        const qk::PassStageIn &pi = pp.in[s];
        const size_t xb = (size_t)pp.cols[s] * sizeof(float);
        if ((pi.aux && overlaps(workspace, (size_t)workspace_bytes, pi.aux, xb)) ||
            (pi.norm_w && overlaps(workspace, (size_t)workspace_bytes, pi.norm_w, xb)))
            return fail(QK_EINVAL_PTR, "qk_gemv_pass_create: the workspace overlaps an input");
    }
    int dev = 0;
    const int hs = hip_status(hipGetDevice(&dev), "qk_gemv_pass_create");
    if (hs != QK_OK) return hs;
    const int G = qk::pass_grid();
    hipError_t he = hipSuccess;
    const int b = qk::pass_build(pp.items.data(), n, pp.first.data(), S, pp.cols.data(), pp.in.data(),
                                 pp.chained.data(), G, workspace, &he);
    if (b == -1) return fail(QK_EINVAL_SHAPE, "qk_gemv_pass_create: a stage's rows do not fit its workgroups");
    if (b != 0) return hip_status(he, "qk_gemv_pass_create: writing the workspace");
    qk_gemv_pass *p = new (std::nothrow) qk_gemv_pass{workspace, S, G, dev, int64_t(1) << 16};
    if (!p) return fail(QK_ENOMEM, "qk_gemv_pass_create: out of host memory");
    *out = p;
    return QK_OK;
}

int qk_gemv_pass_run(const qk_gemv_pass *p, void *stream) {
    g_err[0] = 0;
    if (!p) return fail(QK_EINVAL_PTR, "qk_gemv_pass_run: NULL pass");
    int dev = 0;
    const int hs = hip_status(hipGetDevice(&dev), "qk_gemv_pass_run");
    if (hs != QK_OK) return hs;
    if (dev != p->device) return fail(QK_EINVAL_PTR, "qk_gemv_pass_run: the pass was created on another device");
    return hip_status(qk::pass_launch(p->ws, p->nstages, p->grid, p->spin_limit, (hipStream_t)stream),
                      "qk_gemv_pass_run launch");
}

int qk_gemv_pass_set_spin_limit(qk_gemv_pass *p, int64_t polls) {
    if (!p) return fail(QK_EINVAL_PTR, "qk_gemv_pass_set_spin_limit: NULL pass");
    if (polls < 0) return fail(QK_EINVAL_SHAPE, "qk_gemv_pass_set_spin_limit: negative limit");
    p->spin_limit = polls;
    return QK_OK;
}

int qk_gemv_pass_gave_up(const qk_gemv_pass *p) {
    if (!p) return fail(QK_EINVAL_PTR, "qk_gemv_pass_gave_up: NULL pass");
    uint32_t e = 0;
    const int hs = hip_status(qk::pass_last_error(p->ws, &e), "qk_gemv_pass_gave_up");
    return hs != QK_OK ? hs : (e != 0 ? 1 : 0);
}

int qk_gemv_pass_grid(const qk_gemv_pass *p) { return p ? p->grid : fail(QK_EINVAL_PTR, "NULL pass"); }

void qk_gemv_pass_destroy(qk_gemv_pass *p) { delete p; }

int qk_gemv_kernel_path(int type, int64_t rows, int64_t cols) {
    const FormatInfo *f = format_of(type);
    if (!f) return QK_EINVAL_TYPE;
    if (rows < 1 || cols < 1 || cols % f->elems) return QK_EINVAL_SHAPE;
    return qk::gemv_path(type, rows, cols);
}

int qk_gemm_kernel_path(int type, int64_t rows, int64_t cols, int64_t M) {
    const FormatInfo *f = format_of(type);
    if (!f) return QK_EINVAL_TYPE;
    if (rows < 1 || cols < 1 || cols % f->elems || M < 1) return QK_EINVAL_SHAPE;
    return qk::gemm_path(type, rows, cols, M);
}

int qk_gemv_input_supported(int type, int64_t rows, int64_t cols) {
    const FormatInfo *f = format_of(type);
    if (!f || rows < 1 || cols < 1 || cols % f->elems) return 0;
    return qk::gemv_input_ok(type, rows, cols) ? 1 : 0;
}

int qk_gemv_batch_input(const qk_gemv_desc *descs, int n, const qk_gemv_input *in, void *stream) {
    g_err[0] = 0;
    if (n < 1 || n > qk::kGemvMaxMats) return fail(QK_EINVAL_SHAPE, "qk_gemv_batch_input: 1 to 4 GEMVs");
    if (!descs || !in) return fail(QK_EINVAL_PTR, "qk_gemv_batch_input: descs or in is NULL");
    if (in->kind < QK_INPUT_PLAIN || in->kind > QK_INPUT_SWIGLU) return fail(QK_EINVAL_TYPE, "unknown input kind");
    const qk_gemv_desc &d0 = descs[0];
    for (int i = 0; i < n; i++) {
        const qk_gemv_desc &d = descs[i];
        const int st = check_desc(d);
        if (st != QK_OK) return st;
        if (d.rows < 1 || d.cols != d0.cols || d.x != d0.x || d.cols < 1)
            return fail(QK_EINVAL_SHAPE, "qk_gemv_batch_input: every GEMV needs rows, and the same cols and x");
        if (!qk::gemv_input_ok(d.type, d.rows, d.cols) || !qk::gemv_groupable(d.type, d0.type))
            return fail(QK_EINVAL_SHAPE, "qk_gemv_batch_input: a format or shape without a transformed-input kernel "
                                         "(see qk_gemv_input_supported) or formats that do not share a launch");
    }
    const size_t xb = (size_t)d0.cols * sizeof(float);
    if (in->kind != QK_INPUT_PLAIN) {
        if (!in->aux) return fail(QK_EINVAL_PTR, "qk_gemv_batch_input: aux is NULL");
        if (!aligned(in->aux, 16)) return fail(QK_EALIGN, "qk_gemv_batch_input: aux must be 16-byte aligned");
    }
    if (in->kind == QK_INPUT_ADD_RMSNORM) {
        if (!in->norm_w || !in->x_out) return fail(QK_EINVAL_PTR, "qk_gemv_batch_input: norm_w or x_out is NULL");
        if (!aligned(in->norm_w, 16) || !aligned(in->x_out, 16))
            return fail(QK_EALIGN, "qk_gemv_batch_input: norm_w and x_out must be 16-byte aligned");
        if (overlaps(in->x_out, xb, d0.x, xb) || overlaps(in->x_out, xb, in->aux, xb) ||
            overlaps(in->x_out, xb, in->norm_w, xb))
            return fail(QK_EINVAL_PTR, "qk_gemv_batch_input: x_out overlaps x, aux or norm_w");
    }
    for (int i = 0; i < n; i++) {
        const qk_gemv_desc &a = descs[i];
        const size_t ny = (size_t)a.rows * sizeof(float);
        if ((in->kind != QK_INPUT_PLAIN && overlaps(a.y, ny, in->aux, xb)) ||
            (in->kind == QK_INPUT_ADD_RMSNORM && (overlaps(a.y, ny, in->x_out, xb) || overlaps(a.y, ny, in->norm_w, xb))))
            return fail(QK_EINVAL_PTR, "qk_gemv_batch_input: an output overlaps an input");
        for (int j = 0; j < n; j++) {
            const qk_gemv_desc &b = descs[j];
            const size_t wb = (size_t)(b.rows * qk_row_bytes(b.type, b.cols));
            if ((j != i && overlaps(a.y, ny, b.y, (size_t)b.rows * sizeof(float))) || overlaps(a.y, ny, b.W, wb) ||
                overlaps(a.y, ny, b.x, xb))
                return fail(QK_EINVAL_PTR, "an output overlaps another output or an input of the batch");
        }
    }
    qk::GemvItem items[qk::kGemvMaxMats];
    for (int i = 0; i < n; i++) items[i] = qk::GemvItem{descs[i].type, descs[i].W, descs[i].rows, descs[i].y};
    const qk::GemvInput xin{in->kind, in->aux, in->norm_w, in->eps, in->x_out};
    return hip_status(qk::launch_gemv_group(items, n, d0.cols, d0.x, (hipStream_t)stream, &xin),
                      "qk_gemv_batch_input launch");
}

int qk_gemm_prefill(int type, const void *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M, float *Y,
                    void *stream) {
    g_err[0] = 0;
    int64_t rb = 0;
    const int st = check_matrix(type, W, rows, cols, &rb);
    if (st != QK_OK) return st;
    if (M < 0) return fail(QK_EINVAL_SHAPE, "negative M");
    if (M > 0 && rows > INT64_MAX / M) return fail(QK_EINVAL_SHAPE, "output size overflows");
    if (rows == 0 || M == 0) return QK_OK;
    if (!Y) return fail(QK_EINVAL_PTR, "Y is NULL");
    if (!aligned(Y, 4)) return fail(QK_EALIGN, "Y must be 4-byte aligned");
    if (cols == 0) return hip_status(qk::launch_fill_zero(Y, rows * M, (hipStream_t)stream), "gemm launch");
    if (check_weights_ptr(W) != QK_OK) return check_weights_ptr(W);
    if (!X) return fail(QK_EINVAL_PTR, "X is NULL");
    if (!aligned(X, 16)) return fail(QK_EALIGN, "X must be 16-byte aligned");
    if (cols > INT64_MAX / 2 / M) return fail(QK_EINVAL_SHAPE, "X size overflows");
    // Y may be zeroed before the products are added into it
    const size_t ny = (size_t)(M * rows) * sizeof(float);
    if (overlaps(Y, ny, W, (size_t)(rows * rb)) || overlaps(Y, ny, X, (size_t)(M * cols) * sizeof(uint16_t)))
        return fail(QK_EINVAL_PTR, "Y overlaps W or X");
    return hip_status(qk::launch_gemm(type, W, rows, cols, X, M, Y, (hipStream_t)stream), "gemm launch");
}

}  // extern "C"
