// qk_gemv.hip — the GEMV kernels (one launch per matrix or per group of
// matrices that share x) and their launchers: plan, grid and read mode per
// format and shape. The device code is in qk_gemv_body.h.
#include "qk_gemv_body.h"

namespace qk {

// One launch over the matrices of w: F1 for matrices [0, n1), F2 for the
// rest (F1 == F2: one format).
template <int F1, int F2, int DEPTH, bool SPLIT, bool WIDE, int SPL, int XF = 0>
__global__ __launch_bounds__(256) void gemv_kernel(GemvWork w, GemvPlan p) {
    extern __shared__ __attribute__((aligned(16))) float res[];
    const MatSel ms = mat_sel(w, p, (int)blockIdx.x);
    if constexpr (F1 == F2) {
        gemv_body<F1, DEPTH, SPLIT, WIDE, SPL, XF>(w.x, ms, res, w.in);
    } else {
        if (ms.j == 0)
            gemv_body<F1, DEPTH, SPLIT, WIDE, SPL, XF>(w.x, ms, res, w.in);
        else
            gemv_body<F2, DEPTH, SPLIT, WIDE, SPL, XF>(w.x, ms, res, w.in);
    }
}

// Rows wider than kRegStageCols: rows split over up to 8 waves (512 lanes),
// x staged in rounds (its LDS copy may exceed 64 KiB on gfx950).
template <int F1, int F2, int XF>
__global__ __launch_bounds__(512) void gemv_wide_kernel(GemvWork w, GemvPlan p) {
    extern __shared__ __attribute__((aligned(16))) float res[];
    const MatSel ms = mat_sel(w, p, (int)blockIdx.x);
    if constexpr (F1 == F2) {
        gemv_body<F1, 2, true, true, 0, XF, true>(w.x, ms, res, w.in);
    } else {
        if (ms.j == 0)
            gemv_body<F1, 2, true, true, 0, XF, true>(w.x, ms, res, w.in);
        else
            gemv_body<F2, 2, true, true, 0, XF, true>(w.x, ms, res, w.in);
    }
}

// Generic path: any block count per row, any 2-byte aligned rows, any cols.
// One wave per row; lanes walk the row four weights at a time with the
// bit-exact decoder.
template <int F>
__global__ __launch_bounds__(256) void gemv_generic_kernel(const uint8_t *__restrict__ W, int64_t rows, int64_t cols,
                                                           int64_t row_bytes, const float *__restrict__ x,
                                                           float *__restrict__ y) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t r = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); r < rows; r += nwaves) {
        const uint8_t *row = W + r * row_bytes;
        float acc = 0.f;
        for (int64_t c = 4 * (int64_t)lane; c < cols; c += 256) {
            float w[4];
            decode4<F>(row + (c / QK) * BYTES, (int)(c % QK), w);
            acc += w[0] * x[c] + w[1] * x[c + 1] + w[2] * x[c + 2] + w[3] * x[c + 3];
        }
        for (int m = 32; m > 0; m >>= 1) acc += __shfl_xor(acc, m);
        if (lane == 0) y[r] = acc;
    }
}


// Launch over the n matrices of w (G[j] row groups each), sizing the grid
// from the occupancy. XLOOP: the wide-row kernel.
template <int F1, int F2, bool SPLIT, int DEPTH, bool WIDE, int SPL, int XF = 0, bool XLOOP = false>
static hipError_t launch_fast(GemvWork &w, const GemvPlan &p, const int64_t *G, int n, int np, hipStream_t stream) {
    const int threads = 64 * p.KS * p.NWR;
    const int64_t RG = p.NWR * p.RP;
    static_assert(!XLOOP || (SPLIT && WIDE && DEPTH == 2 && SPL == 0), "the wide-row kernel's configuration");
    const auto kern = XLOOP ? gemv_wide_kernel<F1, F2, XF> : gemv_kernel<F1, F2, DEPTH, SPLIT, WIDE, SPL, XF>;
    // Workgroups resident per CU for this kernel (cached per device and
    // configuration), taken with the largest LDS a workgroup may use; for
    // wide rows the LDS depends on the width and is taken as it is.
    const int64_t lds = XLOOP ? x_lds_floats((int64_t)p.U * Unit<F1>::W) + kMaxRes : 6528 + 384 + kMaxRes;
    if (XLOOP && lds * (int64_t)sizeof(float) > 65536) {
        // more than 64 KiB of dynamic LDS (set once per device)
        const hipError_t e = allow_max_dynamic_lds(reinterpret_cast<const void *>(kern));
        if (e != hipSuccess) return e;
    }
    const int o = occupancy(reinterpret_cast<const void *>(kern), threads, (size_t)lds * sizeof(float));
    // Workgroups per CU: two for launches that give each workgroup only a
    // few row groups (the decode shapes, lm_head included: fewer, longer-lived
    // waves amortise the x staging); four when every workgroup streams many
    // row groups, so that more loads are in flight (workgroups beyond the
    // resident ones start as others finish, which also evens out the tail).
    // Measured on the decode shapes and on >= 1 GiB GEMVs at 2048 and 5632
    // columns (QK_TUNE_GEMV_WGS_PER_CU overrides).
    const int cus = device_cu_count();
    int64_t total_groups = 0;
    for (int j = 0; j < n; j++) total_groups += G[j];
    const int dflt = total_groups > (int64_t)16 * cus ? 4 : (o < 2 ? o : 2);
    const int per_cu = tuning(QK_TUNE_GEMV_WGS_PER_CU) > 0 ? tuning(QK_TUNE_GEMV_WGS_PER_CU) : dflt;
    const int64_t slots = (int64_t)cus * (per_cu > 0 ? per_cu : o);
    // Workgroups per matrix: one per row group while they all fit, else in
    // proportion to the matrices' bytes (at least one each).
    int64_t wg[kMaxMats] = {0, 0, 0, 0};
    const int64_t total = total_groups;
    double bytes = 0.0;
    for (int j = 0; j < n; j++) bytes += (double)G[j] * w.row_bytes[j < w.n1 ? 0 : 1];
    for (int j = 0; j < n; j++) {
        if (total <= slots) {
            wg[j] = G[j];
        } else {
            const double bj = (double)G[j] * w.row_bytes[j < w.n1 ? 0 : 1];
            wg[j] = (int64_t)((double)slots * bj / bytes);
            wg[j] = wg[j] < 1 ? 1 : (wg[j] > G[j] ? G[j] : wg[j]);
        }
        if (SPLIT) {
            // every workgroup's rows (times KS partials) must fit the result buffer
            const int64_t mn = (G[j] * RG * p.KS + kMaxRes - 1) / kMaxRes;
            if (wg[j] < mn) wg[j] = mn;
        }
    }
    int64_t maxg = 0, grid = 0;  // most groups of one workgroup; workgroups
    for (int j = 0; j < kMaxMats; j++) {
        w.wgbeg[j] = (int)grid;
        if (j < n) {
            w.q[j] = (int)(G[j] / wg[j]);
            w.r[j] = (int)(G[j] % wg[j]);
            const int64_t mg = (G[j] + wg[j] - 1) / wg[j];
            if (mg > maxg) maxg = mg;
            grid += wg[j];
        } else {
            w.q[j] = w.r[j] = 0;
        }
    }
    for (int j = n; j < kMaxMats; j++) w.wgbeg[j] = (int)grid;
    const int64_t cols = (int64_t)p.U * Unit<F1>::W;
    // LDS: x and its sums (in the streamed mode also the two group slots,
    // 16-byte aligned, over the same space), then the KS partial results
    const size_t x_fl = (size_t)((cols + 4 * (cols / 64) + cols / 16 + 3) & ~(int64_t)3);
    const size_t lead = SPL > 0 && (size_t)(8 * np) > x_fl ? (size_t)(8 * np) : x_fl;
    const size_t shmem = (lead + (p.KS > 1 ? (size_t)(maxg * RG * p.KS) : 0)) * sizeof(float);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(threads), shmem, stream, w, p);
    return hipGetLastError();
}



// Streamed mode (rows not split over waves): a group of row slots per wave
// reads its rows from LDS.
template <int F1, int F2, int SPL>
static hipError_t launch_stream(GemvWork &w, const GemvPlan &p, const int64_t *G, int n, int np, hipStream_t stream) {
    return p.Lshift >= 4 ? launch_fast<F1, F2, false, 2, true, SPL>(w, p, G, n, np, stream)
                         : launch_fast<F1, F2, false, 2, false, SPL>(w, p, G, n, np, stream);
}

// Launches of at least this many weight bytes use the streamed mode: below
// it the fill and drain of the two-group pipeline cost more than the
// streaming gains (measured on Q4_K, Q6_K and q8_0 GEMVs of 16 MiB to 1 GiB
// at 2048 columns: the streamed mode is ahead from 128 MiB on).
constexpr int64_t kStreamMinBytes = int64_t(128) << 20;

// How a group of GEMVs of one width runs in the fused kernels: wide rows
// (more than kRegStageCols columns), or streamed through LDS, or direct.
// Streamed mode: each row group is read as one contiguous stream of 16-byte
// pieces through LDS. It needs every matrix to be a whole number of 16-byte
// pieces (its last piece is read whole) and a group of at most 4 pieces per
// thread. It is used for rows that one wave covers (with rows split over
// waves its two-row groups keep too few bytes in flight), not for q4_0,
// whose small groups measured slower streamed, and not with a transformed
// input; by default for launches of at least kStreamMinBytes.
// QK_TUNE_GEMV_STREAM = 0/1 forces it off/on where it applies.
struct GroupMode {
    bool wide, streamed;
    int np, spl;  // streamed mode: 16-byte pieces per row group, pieces per thread
};
template <int F1, int F2>
static GroupMode group_mode(const GemvPlan &p, int64_t cols, const GemvItem *items, int n, int n1, int kind) {
    GroupMode m{cols > kRegStageCols, false, 0, 0};
    const int64_t RG = p.NWR * p.RP;
    const int threads = 64 * p.KS * p.NWR;
    const int64_t rb1 = cols / Layout<F1>::QK * Layout<F1>::BYTES, rb2 = cols / Layout<F2>::QK * Layout<F2>::BYTES;
    int64_t np = 0, bytes = 0;
    bool ok = p.KS == 1 && F1 != Q4_0 && kind == 0;
    for (int j = 0; j < n; j++) {
        const int64_t rb = j < n1 ? rb1 : rb2;
        const int64_t npj = (RG * rb + 159) / 16;
        np = npj > np ? npj : np;
        bytes += items[j].rows * rb;
        if ((items[j].rows * rb) % 16 != 0) ok = false;
    }
    const int spl = (int)((np + threads - 1) / threads);
    const int64_t x_fl = cols + 4 * (cols / 64) + cols / 16 + 4;
    const int64_t lds_fl = (8 * np > x_fl ? 8 * np : x_fl) + 2048;  // partial results <= 2048 floats
    if (spl > 4 || lds_fl * 4 > 65536) ok = false;
    const int force = tuning(QK_TUNE_GEMV_STREAM);
    m.streamed = !m.wide && ok && (force < 0 ? bytes >= kStreamMinBytes : force > 0);
    m.np = (int)np;
    m.spl = spl;
    return m;
}

// items[0..n1) have format F1, items[n1..n) format F2.
template <int F1, int F2>
static hipError_t launch_group_t(const GemvItem *items, int n, int n1, int64_t cols, const float *x,
                                 hipStream_t stream, const GemvInput *xin) {
    static_assert(Unit<F1>::W == Unit<F2>::W && Layout<F1>::QK == Layout<F2>::QK, "formats must share a plan");
    const GemvPlan p = make_plan<F1>(cols);
    const int64_t RG = p.NWR * p.RP;
    GemvWork w;
    w.x = x;
    w.in = xin ? *xin : GemvInput{0, nullptr, nullptr, 0.f, nullptr};
    w.W = static_cast<const uint8_t *>(items[0].W);
    w.y = items[0].y;
    int64_t G[kMaxMats] = {0, 0, 0, 0};
    for (int j = 0; j < kMaxMats; j++) {
        const bool used = j < n;
        w.wof[j] = used ? (int64_t)((uintptr_t)items[j].W - (uintptr_t)items[0].W) : 0;
        w.yof[j] = used ? (int64_t)(((uintptr_t)items[j].y - (uintptr_t)items[0].y) / sizeof(float)) : 0;
        w.rows[j] = used ? (int)items[j].rows : 1;
        if (used) G[j] = (items[j].rows + RG - 1) / RG;
    }
    w.n1 = n1;
    w.row_bytes[0] = (int)(cols / Layout<F1>::QK * Layout<F1>::BYTES);
    w.row_bytes[1] = (int)(cols / Layout<F2>::QK * Layout<F2>::BYTES);
    // Two row buffers per wave (one row's loads in flight while another is
    // decoded): a third buffer measured no better on long launches and worse
    // where it cost occupancy (Q6_K rows split over waves).
    const GroupMode m = group_mode<F1, F2>(p, cols, items, n, n1, w.in.kind);
    if (m.wide) {
        // wide rows (always split over waves): x staged in rounds
        if (w.in.kind == 0) return launch_fast<F1, F2, true, 2, true, 0, 0, true>(w, p, G, n, 0, stream);
        if constexpr ((F1 == Q4_K || F1 == Q6_K || F1 == Q4_0 || F1 == Q8_0) &&
                      (F2 == Q4_K || F2 == Q6_K || F2 == Q4_0 || F2 == Q8_0)) {
            return w.in.kind == 1 ? launch_fast<F1, F2, true, 2, true, 0, 1, true>(w, p, G, n, 0, stream)
                                  : launch_fast<F1, F2, true, 2, true, 0, 2, true>(w, p, G, n, 0, stream);
        }
        return hipErrorInvalidValue;
    }
    if (w.in.kind != 0) {
        // transformed inputs: the direct mode, in the K-quant and the
        // q4_0/q8_0 families only
        if constexpr ((F1 == Q4_K || F1 == Q6_K || F1 == Q4_0 || F1 == Q8_0) &&
                      (F2 == Q4_K || F2 == Q6_K || F2 == Q4_0 || F2 == Q8_0)) {
            if (w.in.kind == 1) {
                if (p.KS > 1) return launch_fast<F1, F2, true, 2, true, 0, 1>(w, p, G, n, 0, stream);
                return p.Lshift >= 4 ? launch_fast<F1, F2, false, 2, true, 0, 1>(w, p, G, n, 0, stream)
                                     : launch_fast<F1, F2, false, 2, false, 0, 1>(w, p, G, n, 0, stream);
            }
            if (p.KS > 1) return launch_fast<F1, F2, true, 2, true, 0, 2>(w, p, G, n, 0, stream);
            return p.Lshift >= 4 ? launch_fast<F1, F2, false, 2, true, 0, 2>(w, p, G, n, 0, stream)
                                 : launch_fast<F1, F2, false, 2, false, 0, 2>(w, p, G, n, 0, stream);
        }
        return hipErrorInvalidValue;
    }
    if (!m.streamed) {
        if (p.KS > 1) return launch_fast<F1, F2, true, 2, true, 0>(w, p, G, n, 0, stream);
        return p.Lshift >= 4 ? launch_fast<F1, F2, false, 2, true, 0>(w, p, G, n, 0, stream)
                             : launch_fast<F1, F2, false, 2, false, 0>(w, p, G, n, 0, stream);
    }
    switch (m.spl) {
    case 1: return launch_stream<F1, F2, 1>(w, p, G, n, m.np, stream);
    case 2: return launch_stream<F1, F2, 2>(w, p, G, n, m.np, stream);
    case 3: return launch_stream<F1, F2, 3>(w, p, G, n, m.np, stream);
    default: return launch_stream<F1, F2, 4>(w, p, G, n, m.np, stream);
    }
}

template <int F>
static hipError_t launch_generic_t(const uint8_t *W, int64_t rows, int64_t cols, const float *x, float *y,
                                   hipStream_t stream) {
    const int64_t row_bytes = cols / Layout<F>::QK * Layout<F>::BYTES;
    int64_t grid = (rows + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 8;
    if (grid > cap) grid = cap;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(gemv_generic_kernel<F>, dim3((unsigned)grid), dim3(256), 0, stream, W, rows, cols, row_bytes,
                       x, y);
    return hipGetLastError();
}

bool gemv_fusable(int type, int64_t rows, int64_t cols) {
    switch (type) {
    case Q4_K: return fast_ok<Q4_K>(rows, cols);
    case Q6_K: return fast_ok<Q6_K>(rows, cols);
    case Q8_0: return fast_ok<Q8_0>(rows, cols);
    case Q4_0: return fast_ok<Q4_0>(rows, cols);
    case Q8_0_F16: return fast_ok<Q8_0_F16>(rows, cols);
    case Q5_1: return fast_ok<Q5_1>(rows, cols);
    case Q5_K: return fast_ok<Q5_K>(rows, cols);
    case Q2_K: return fast_ok<Q2_K>(rows, cols);
    case Q3_K: return fast_ok<Q3_K>(rows, cols);
    default: return false;
    }
}

// Formats whose GEMVs share a launch: Q4_K with Q6_K and q4_0 with q8_0
// (same unit and block size); each other format only with itself.
static int family(int type) {
    return (type == Q4_K || type == Q6_K) ? 1 : (type == Q4_0 || type == Q8_0) ? 2 : 100 + type;
}

bool gemv_groupable(int a, int b) { return family(a) == family(b); }

bool gemv_input_ok(int type, int64_t rows, int64_t cols) {
    return gemv_fusable(type, rows, cols) && (family(type) == 1 || family(type) == 2);
}

template <int F> static int path_t(int64_t rows, int64_t cols) {
    const GemvItem it{F, nullptr, rows, nullptr};
    const GroupMode m = group_mode<F, F>(make_plan<F>(cols), cols, &it, 1, 1, 0);
    return m.wide ? 3 : m.streamed ? 2 : 1;
}

int gemv_path(int type, int64_t rows, int64_t cols) {
    if (!gemv_fusable(type, rows, cols)) return 0;
    switch (type) {
    case Q4_K: return path_t<Q4_K>(rows, cols);
    case Q6_K: return path_t<Q6_K>(rows, cols);
    case Q8_0: return path_t<Q8_0>(rows, cols);
    case Q4_0: return path_t<Q4_0>(rows, cols);
    case Q8_0_F16: return path_t<Q8_0_F16>(rows, cols);
    case Q5_1: return path_t<Q5_1>(rows, cols);
    case Q5_K: return path_t<Q5_K>(rows, cols);
    case Q2_K: return path_t<Q2_K>(rows, cols);
    case Q3_K: return path_t<Q3_K>(rows, cols);
    default: return 0;
    }
}

hipError_t launch_gemv_group(const GemvItem *items, int n, int64_t cols, const float *x, hipStream_t stream,
                             const GemvInput *xin) {
    if (n < 1 || n > kGemvMaxMats) return hipErrorInvalidValue;
    // first format: Q6_K or q4_0 when present; its items go first (Q6_K
    // first: its rows take longer per row group than Q4_K's, and its
    // workgroups then start first; the 1.1B decode pass's q/k/v launch
    // 4.12 -> 3.93 us, the pass 0.426 -> 0.424 ms)
    const int fam = family(items[0].type);
    const int first = fam == 1 ? Q6_K : fam == 2 ? Q4_0 : items[0].type;
    const int second = fam == 1 ? Q4_K : fam == 2 ? Q8_0 : items[0].type;
    GemvItem sorted[kGemvMaxMats];
    int n1 = 0, k = 0;
    for (int i = 0; i < n; i++) {
        if (family(items[i].type) != fam) return hipErrorInvalidValue;
        if (items[i].type == first && items[i].rows > 0) sorted[k++] = items[i];
    }
    n1 = k;
    if (second != first)
        for (int i = 0; i < n; i++)
            if (items[i].type == second && items[i].rows > 0) sorted[k++] = items[i];
    n = k;  // matrices with rows
    if (n == 0) return hipSuccess;
    if (n1 == 0 || n1 == n) {
        switch (sorted[0].type) {
        case Q4_K: return launch_group_t<Q4_K, Q4_K>(sorted, n, n, cols, x, stream, xin);
        case Q6_K: return launch_group_t<Q6_K, Q6_K>(sorted, n, n, cols, x, stream, xin);
        case Q8_0: return launch_group_t<Q8_0, Q8_0>(sorted, n, n, cols, x, stream, xin);
        case Q4_0: return launch_group_t<Q4_0, Q4_0>(sorted, n, n, cols, x, stream, xin);
        case Q8_0_F16: return launch_group_t<Q8_0_F16, Q8_0_F16>(sorted, n, n, cols, x, stream, xin);
        case Q5_1: return launch_group_t<Q5_1, Q5_1>(sorted, n, n, cols, x, stream, xin);
        case Q5_K: return launch_group_t<Q5_K, Q5_K>(sorted, n, n, cols, x, stream, xin);
        case Q2_K: return launch_group_t<Q2_K, Q2_K>(sorted, n, n, cols, x, stream, xin);
        case Q3_K: return launch_group_t<Q3_K, Q3_K>(sorted, n, n, cols, x, stream, xin);
        default: return hipErrorInvalidValue;
        }
    }
    return fam == 1 ? launch_group_t<Q6_K, Q4_K>(sorted, n, n1, cols, x, stream, xin)
                    : launch_group_t<Q4_0, Q8_0>(sorted, n, n1, cols, x, stream, xin);
}

hipError_t launch_gemv(int type, const void *W, int64_t rows, int64_t cols, const float *x, float *y,
                       hipStream_t stream) {
    if (gemv_fusable(type, rows, cols)) {
        const GemvItem it{type, W, rows, y};
        return launch_gemv_group(&it, 1, cols, x, stream);
    }
    const uint8_t *w = static_cast<const uint8_t *>(W);
    switch (type) {
    case Q4_K: return launch_generic_t<Q4_K>(w, rows, cols, x, y, stream);
    case Q6_K: return launch_generic_t<Q6_K>(w, rows, cols, x, y, stream);
    case Q8_0: return launch_generic_t<Q8_0>(w, rows, cols, x, y, stream);
    case Q4_0: return launch_generic_t<Q4_0>(w, rows, cols, x, y, stream);
    case Q8_0_F16: return launch_generic_t<Q8_0_F16>(w, rows, cols, x, y, stream);
    case Q5_1: return launch_generic_t<Q5_1>(w, rows, cols, x, y, stream);
    case Q5_K: return launch_generic_t<Q5_K>(w, rows, cols, x, y, stream);
    case Q2_K: return launch_generic_t<Q2_K>(w, rows, cols, x, y, stream);
    case Q3_K: return launch_generic_t<Q3_K>(w, rows, cols, x, y, stream);
    default: return hipErrorInvalidValue;
    }
}

__global__ void fill_zero_kernel(float *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0.f;
}

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream) {
    int64_t grid = (n + 255) / 256;
    if (grid > 4096) grid = 4096;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)grid), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

}  // namespace qk
