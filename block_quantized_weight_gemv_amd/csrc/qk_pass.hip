// qk_pass.hip — a whole decode-step weight pass in one persistent launch.
//
// The pages' forward pass runs the projections of a layer in a fixed order,
// each stage reading an x computed from what the stage before produced
// ("picoLM, in Python", §4 — The forward pass: q, k and v read one normed x,
// o the attention output, gate and up another normed x, down the SwiGLU
// product). On this GPU a launch per stage costs more than the stage's own
// weight traffic at 1.1B shapes (an empty kernel in a graph takes ~1.7 us, a
// stage streams 3-13 MB in 0.5-2 us), so here one launch walks all the
// stages, and a stage starts as soon as the data it reads exists.
//
// * One workgroup per CU, all resident, of seven waves. Waves 1-6 decode:
//   in stage s each takes its rows of the workgroup's share with the same
//   lane plan, decode and reduction as a per-stage launch of the same
//   matrices (the same bits). Wave 0 writes the stage's y.
// * The compute waves request the weights of their first row groups of a
//   stage before they read its x: weights never depend on an earlier stage,
//   so they stream in while x is still being produced.
// * Flagged data instead of barriers: an output that a later stage reads is
//   also written to a mirror in the workspace as 8-byte words {value bits,
//   run epoch}, one store each. A consumer reads x straight from the mirror
//   and takes a word once its epoch is the current run's; a word whose epoch
//   is older is read again. The value and its flag travel in one store, so
//   nothing waits for stores to complete and no counter is needed (a
//   counter protocol costs a store acknowledgement, an atomic, a poll and
//   the x load, each a device-wide round trip of ~0.9 us). Mirror words are
//   written and read with device-scope (sc1) accesses, which are coherent
//   across the XCDs' L2 caches.
// * Splitting the roles keeps each wave's load counter free of the other
//   role's traffic (the counter is in-order over loads and stores): wave 0
//   never waits for its stores, and the compute waves wait for each row
//   group's loads without waiting for stores.
// * The input transform of a stage (RMSNorm, SwiGLU) is applied as x is
//   staged in LDS; RMSNorm's sum of squares is taken over all of x by every
//   workgroup.
// * Every wait is bounded: past a spin limit a wait sets an error word and
//   goes on with what it read (the results are then not to be trusted, but
//   the launch ends). After the last stage each workgroup counts itself out;
//   the last one advances the run epoch and records the error word.
#include <cstring>
#include <vector>

#include "qk_gemv_body.h"

namespace qk {

constexpr int kPassIo = 1;                                   // the wave that writes y
constexpr int kPassCompute = 6;                              // compute waves (row plans of 1, 2 or 3 waves per row)
constexpr int kPassThreads = 64 * (kPassIo + kPassCompute);
constexpr int kPassBufs = 4;                                 // row groups of weights in flight per lane
constexpr int kPassChunks = 4;                               // 16-byte chunks of x per compute thread
static_assert(kPassChunks * 64 * kPassCompute * 4 >= kRegStageCols, "one round of chunks stages the widest x");

// The words at the start of the workspace.
enum { kPassErr = 0, kPassLastErr = 1, kPassExits = 2, kPassEpoch = 3, kPassHeadWords = 32 };

struct PassStage {
    GemvWork w;   // the stage's matrices (w.x: x when read from memory)
    GemvPlan p;   // NWR = kPassCompute / KS
    int f1, f2;   // formats of matrices [0, n1) and [n1, n)
    int split;    // rows split over waves
    int wide;     // row slots of 16 or more lanes
    int nwg;      // workgroups with rows in this stage
    int kind;     // input transform: 0 x, 1 RMSNorm(x) (* norm_w), 2 silu(x) * aux
    float eps;
    int pad0;
    int64_t x_ll;             // mirror word of x[0], or -1: x read from memory
    int64_t aux_ll;           // the same for aux
    const float *aux;         // aux when read from memory
    const float *norm_w;      // or nullptr (weights of 1)
    int64_t y_ll[kMaxMats];   // mirror word of each matrix's y[0], or -1: no later stage reads it
};

// LDS of a pass workgroup: x (up to kRegStageCols columns, padded) and its
// sums, then the row results (KS partials per row).
constexpr int kPassXFloats = (kRegStageCols + 4 * (kRegStageCols / 64) + kRegStageCols / 16 + 3) & ~3;
constexpr int64_t kPassLdsFloats = kPassXFloats + kMaxRes;

// Pointers read from the stage table are generic to the compiler; these
// views make their loads and stores global-memory instructions (a generic
// load also counts on the LDS counter, and the waits for it cannot be
// exact).
#define QK_GLOBAL __attribute__((address_space(1)))
typedef const QK_GLOBAL uint8_t *gbytes;
typedef uint32_t u32x4_ga4 __attribute__((ext_vector_type(4), aligned(4)));

__device__ __forceinline__ u32x4 gld_b128(gbytes p) {
    const u32x4_ga4 v = *reinterpret_cast<const QK_GLOBAL u32x4_ga4 *>(p);
    return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ uint32_t gld_b32(gbytes p) { return *reinterpret_cast<const QK_GLOBAL uint32_t *>(p); }
__device__ __forceinline__ float4 gld_f4(const QK_GLOBAL float *p) {
    const u32x4 v = gld_b128(reinterpret_cast<gbytes>(p));
    // (each element through a scalar: this compiler's __builtin_bit_cast of
    // a vector element, e.g. v.y, reads element 0)
    const uint32_t a = v.x, b = v.y, c = v.z, d = v.w;
    return float4{__builtin_bit_cast(float, a), __builtin_bit_cast(float, b), __builtin_bit_cast(float, c),
                  __builtin_bit_cast(float, d)};
}
__device__ __forceinline__ uint32_t gld_b16(gbytes p) { return *reinterpret_cast<const QK_GLOBAL uint16_t *>(p); }

// The raw pieces of unit u of a row, the same bytes into the same fields as
// load_raw (qk_gemv_body.h), through a global view of the row.
template <int F> __device__ __forceinline__ void pass_load(gbytes row, int u, Raw<F> &r);
template <> __device__ __forceinline__ void pass_load<Q4_K>(gbytes row, int u, Raw<Q4_K> &r) {
    const gbytes blk = row + (u >> 2) * 144;
    const int g = u & 3;
    r.h = gld_b128(blk);
    r.qa = gld_b128(blk + 16 + 32 * g);
    r.qb = gld_b128(blk + 32 + 32 * g);
}
template <> __device__ __forceinline__ void pass_load<Q6_K>(gbytes row, int u, Raw<Q6_K> &r) {
    const int h = (u >> 1) & 1, l0 = 16 * (u & 1);
    const gbytes B0 = row + (u >> 2) * 210;
    const uint32_t mis = (uint32_t)(uintptr_t)B0 & 3u;
    const gbytes A0 = B0 - mis;
    r.p[0] = gld_b128(A0 + 64 * h + l0);
    r.p[1] = gld_b128(A0 + 64 * h + 32 + l0);
    r.p[2] = gld_b128(A0 + 128 + 32 * h + l0);
    r.s = gld_b128(A0 + 192);
    r.s4 = gld_b16(B0 + 206) | (gld_b16(B0 + 208) << 16);
    r.e[0] = gld_b32(A0 + 64 * h + l0 + 16);
    r.e[1] = gld_b32(A0 + 64 * h + 32 + l0 + 16);
    r.e[2] = gld_b32(A0 + 128 + 32 * h + l0 + 16);
}

struct PassRun {
    QK_GLOBAL uint64_t *ll;  // the mirror words
    uint32_t ep;             // this run's epoch
    QK_GLOBAL uint32_t *err;
    int64_t limit;           // polls before a wait gives up
};

__device__ __forceinline__ uint64_t ll_load(const QK_GLOBAL uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Chunk c (4 floats) of an input: from memory, or from the mirror (four
// 8-byte device-scope loads), taken once all four words carry the run's
// epoch.
struct XSrc {
    const QK_GLOBAL float *mem;
    const QK_GLOBAL uint64_t *ll;  // nullptr: read from memory
};
__device__ __forceinline__ XSrc make_src(const float *mem, const QK_GLOBAL uint64_t *ll) {
    return XSrc{(const QK_GLOBAL float *)mem, ll};
}
struct XRaw {
    float4 f;
    uint64_t w[4];
};
__device__ __forceinline__ void src_issue(const XSrc &s, int c, XRaw &r) {
    if (s.ll != nullptr) {
#pragma unroll
        for (int k = 0; k < 4; k++) r.w[k] = ll_load(s.ll + 4 * c + k);
    } else {
        r.f = gld_f4(s.mem + 4 * c);
    }
}
__device__ __forceinline__ bool ll_current(const XRaw &r, uint32_t ep) {
    return (uint32_t)(r.w[0] >> 32) == ep && (uint32_t)(r.w[1] >> 32) == ep && (uint32_t)(r.w[2] >> 32) == ep &&
           (uint32_t)(r.w[3] >> 32) == ep;
}
// The value of chunk c: from memory as read, or from the mirror once its
// words are current (read again until they are, or the wait gives up).
__device__ __forceinline__ float4 src_finish(const XSrc &s, int c, XRaw &r, const PassRun &run) {
    if (s.ll == nullptr) return r.f;
    if (run.limit == 0) {  // no polls allowed: every chained read gives up at once
        if ((threadIdx.x & 63) == 0) __hip_atomic_store(run.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        for (int64_t it = 0; !ll_current(r, run.ep); it++) {
            if (it >= run.limit) {
                __hip_atomic_store(run.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            // (once a wait of this run has given up, later ones do not wait;
            // the error word is read only once a wait has lasted 64 polls)
            if (it == 64 && __hip_atomic_load(run.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) break;
            __builtin_amdgcn_s_sleep(1);
            src_issue(s, c, r);
        }
    }
    return float4{__builtin_bit_cast(float, (uint32_t)r.w[0]), __builtin_bit_cast(float, (uint32_t)r.w[1]),
                  __builtin_bit_cast(float, (uint32_t)r.w[2]), __builtin_bit_cast(float, (uint32_t)r.w[3])};
}

// x' for the stage into LDS at the padded positions, with the sums over each
// aligned 16 floats, by the compute waves (thread t = threadIdx.x - 64 takes
// chunks t, t + 384, ...: one round covers 6144 columns); the mirror words
// of all of a thread's chunks are requested before any is checked. For
// RMSNorm the sum of squares is reduced over the workgroup first (one more
// barrier, taken by all waves).
__device__ __forceinline__ void pass_stage_x(const PassStage &st, int cols, float *xs, float *xsum, float *red,
                                             const PassRun &run) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int kind = st.kind;
    const int nch = cols / 4;
    constexpr int NT = 64 * kPassCompute;
    const int t = threadIdx.x - 64 * kPassIo;
    float4 v[kPassChunks];
    if (wave >= kPassIo) {
        const XSrc xsrc = make_src(st.w.x, st.x_ll >= 0 ? run.ll + st.x_ll : nullptr);
        const XSrc asrc = make_src(st.aux, st.aux_ll >= 0 ? run.ll + st.aux_ll : nullptr);
        XRaw rx[kPassChunks], ra[kPassChunks];
        // chunks past the end read the last one again (not stored)
        auto chunk = [&](int i) { return min(t + NT * i, nch - 1); };
#pragma unroll
        for (int i = 0; i < kPassChunks; i++) {
            src_issue(xsrc, chunk(i), rx[i]);
            if (kind == 2) src_issue(asrc, chunk(i), ra[i]);
        }
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < kPassChunks; i++) {
            v[i] = src_finish(xsrc, chunk(i), rx[i], run);
            if (kind == 2) {
                // __expf (v_exp_f32 on g * log2 e) and the hardware reciprocal:
                // a few ulps, inside the GEMV's tolerance
                const float4 a = src_finish(asrc, chunk(i), ra[i], run);
                auto silu_mul = [](float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; };
                v[i] = float4{silu_mul(v[i].x, a.x), silu_mul(v[i].y, a.y), silu_mul(v[i].z, a.z),
                              silu_mul(v[i].w, a.w)};
            }
            if (t + NT * i < nch) ss += v[i].x * v[i].x + v[i].y * v[i].y + v[i].z * v[i].z + v[i].w * v[i].w;
        }
        if (kind == 1) {
            for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
            if (lane == 0) red[wave - kPassIo] = ss;
        }
    }
    float inv = 1.f;
    if (kind == 1) {
        __syncthreads();  // (A0) the sums of squares
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < kPassCompute; i++) tot += red[i];
        inv = 1.0f / sqrtf(tot / (float)cols + st.eps);
    }
    if (wave >= kPassIo) {
        const QK_GLOBAL float *nw = (const QK_GLOBAL float *)st.norm_w;
#pragma unroll
        for (int i = 0; i < kPassChunks; i++) {
            const int c = t + NT * i;
            float4 f = v[i];
            if (kind == 1) {
                f = float4{f.x * inv, f.y * inv, f.z * inv, f.w * inv};
                if (nw != nullptr) {
                    const float4 g = gld_f4(nw + 4 * min(c, nch - 1));
                    f = float4{g.x * f.x, g.y * f.y, g.z * f.z, g.w * f.w};
                }
            }
            float sm = (f.x + f.y) + (f.z + f.w);
            sm = dpp_add<0xB1>(sm);
            sm = dpp_add<0x4E>(sm);
            if (c < nch) {  // uniform over the wave: cols is a multiple of 256
                *reinterpret_cast<float4 *>(xs + xpos(4 * c)) = f;
                if ((c & 3) == 0) xsum[c >> 2] = sm;
            }
        }
    }
}

// One stage of one workgroup whose rows are of format F. The barriers sit at
// the same points for all waves: (A) x is in LDS, (B) the row results are.
template <int F, bool SPLIT, bool WIDE>
__device__ __forceinline__ void pass_stage(const PassStage &st, const MatSel &ms, float *lds, float *red,
                                           const PassRun &run) {
    const GemvPlan &p = ms.p;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int cols = p.U * Unit<F>::W;
    float *const xs = lds;
    float *const xsum = lds + xpos(cols);
    float *const res = lds + kPassXFloats;
    const int RG = p.NWR * p.RP;
    const int g0 = ms.g0, g1 = ms.g1;
    const int nloc = (g1 - g0) * RG;  // rows of this workgroup

    // compute waves: lane plan, as in the per-stage kernel
    const int wc = wave >= kPassIo ? wave - kPassIo : 0;
    const int wr = wc / p.KS;
    const int ks = wc - wr * p.KS;
    const int slot = lane >> p.Lshift, li = lane & ((1 << p.Lshift) - 1);
    const int u_raw = ks * p.Uw + li;
    const bool active = li < p.Uw && u_raw < p.U;
    const int u = active ? u_raw : 0;  // idle lanes read unit 0 and drop it
    const int row_bytes = ms.row_bytes;
    const int rofs = wr * p.RP + slot;
    const int64_t lane_ofs = (int64_t)rofs * row_bytes;
    const int64_t gstride = (int64_t)RG * row_bytes;
    const gbytes Wm = (gbytes)ms.W;  // (a C cast: generic to global)
    const int rows = ms.rows;
    const gbytes last_row = Wm + (int64_t)(rows - 1) * row_bytes;
    auto row_ptr = [&](int g) {
        const int gg = min(g, g1 - 1);
        return gg * RG + rofs < rows ? Wm + gg * gstride + lane_ofs : last_row;
    };

    Raw<F> b[kPassBufs];
    if (wave >= kPassIo) {
        // the first row groups (past the last one: the last one again, so
        // that every lane issues the same loads and the waits stay exact)
#pragma unroll
        for (int d = 0; d < kPassBufs - 1; d++) {
            pass_load<F>(row_ptr(g0 + d), u, b[d]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    pass_stage_x(st, cols, xs, xsum, red, run);
    __syncthreads();  // (A)
    if (wave >= kPassIo) {
        XUnit<F> xu;
        read_x<F>(xs, xsum, u, xu);
        if (!active) {
#pragma unroll
            for (int i = 0; i < Unit<F>::W; i++) xu.v[i] = 0.f;
#pragma unroll
            for (int i = 0; i < Unit<F>::NSUM; i++) xu.s[i] = 0.f;
        }
        auto finish = [&](int g, const Raw<F> &bf) {
            // (dot_raw reads only the alignment of the row's address)
            float part = dot_raw<F>((const uint8_t *)row_ptr(g), u, bf, xu);
            if constexpr (WIDE) {
                part = dpp_add<0xB1>(part);
                part = dpp_add<0x4E>(part);
                part = dpp_add<0x141>(part);
                part = dpp_add<0x140>(part);
                const float t0 = readlane_f(part, 0), t1 = readlane_f(part, 16);
                const float t2 = readlane_f(part, 32), t3 = readlane_f(part, 48);
                const float lo = t0 + t1, hi = t2 + t3;
                const float pair = lane >= 32 ? hi : lo;
                part = p.Lshift == 4 ? part : (p.Lshift == 5 ? pair : lo + hi);
            } else {
                part = reduce16(part, p.Lshift);
            }
            if (li == 0) res[ks * nloc + (g - g0) * RG + rofs] = part;
        };
        int g = g0;
        for (; g + kPassBufs <= g1; g += kPassBufs) {
#pragma unroll
            for (int d = 0; d < kPassBufs; d++) {
                pass_load<F>(row_ptr(g + d + kPassBufs - 1), u, b[(d + kPassBufs - 1) % kPassBufs]);
                __builtin_amdgcn_sched_barrier(0);
                finish(g + d, b[d]);
            }
        }
#pragma unroll
        for (int d = 0; d < kPassBufs - 1; d++)
            if (g + d < g1) finish(g + d, b[d]);
    }
    __syncthreads();  // (B)
    if (wave < kPassIo) {
        // the row results (split rows added in a fixed order) to y, and to
        // its mirror if a later stage reads it; nothing waits for the stores
        QK_GLOBAL float *y = (QK_GLOBAL float *)ms.y;
        const int blk = (int)blockIdx.x;  // its matrix: the workgroup ranges of the stage table
        const int jm = (blk >= st.w.wgbeg[1]) + (blk >= st.w.wgbeg[2]) + (blk >= st.w.wgbeg[3]);
        const int64_t yl = st.y_ll[jm];
        for (int i = threadIdx.x; i < nloc; i += 64 * kPassIo) {
            float sum = res[i];
            if constexpr (SPLIT)
                for (int k = 1; k < p.KS; k++) sum += res[k * nloc + i];
            const int r = g0 * RG + i;
            if (r < rows) {
                y[r] = sum;
                if (yl >= 0)
                    __hip_atomic_store(run.ll + yl + r, ((uint64_t)run.ep << 32) | __builtin_bit_cast(uint32_t, sum),
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

template <int F>
__device__ __forceinline__ void pass_stage_f(const PassStage &st, const MatSel &ms, float *lds, float *red,
                                             const PassRun &run) {
    if (st.split) {
        if (st.wide)
            pass_stage<F, true, true>(st, ms, lds, red, run);
        else
            pass_stage<F, true, false>(st, ms, lds, red, run);
    } else {
        if (st.wide)
            pass_stage<F, false, true>(st, ms, lds, red, run);
        else
            pass_stage<F, false, false>(st, ms, lds, red, run);
    }
}

__global__ __launch_bounds__(kPassThreads) void gemv_pass_kernel(const PassStage *__restrict__ tab, int nstages,
                                                                 uint32_t *head, uint64_t *ll, int64_t limit) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    __shared__ float red[kPassCompute];
    __shared__ uint32_t last;
    QK_GLOBAL uint32_t *const hg = (QK_GLOBAL uint32_t *)head;
    // every workgroup reads the epoch before any has counted itself out
    const PassRun run{(QK_GLOBAL uint64_t *)ll,
                      __hip_atomic_load(hg + kPassEpoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u,
                      hg + kPassErr, limit};
    const int blk = (int)blockIdx.x;
    for (int s = 0; s < nstages; s++) {
        const PassStage &st = tab[s];
        if (blk >= st.nwg) continue;
        const MatSel ms = mat_sel(st.w, st.p, blk);
        if ((ms.j == 0 ? st.f1 : st.f2) == Q4_K)
            pass_stage_f<Q4_K>(st, ms, lds, red, run);
        else
            pass_stage_f<Q6_K>(st, ms, lds, red, run);
    }
    // the last workgroup out advances the epoch for the next run and
    // records the error word (the next run starts after this one has ended)
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(hg + kPassExits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               gridDim.x - 1;
    __syncthreads();
    if (last && threadIdx.x == 0) {
        const uint32_t e = __hip_atomic_load(hg + kPassErr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(hg + kPassLastErr, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(hg + kPassErr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(hg + kPassExits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(hg + kPassEpoch, run.ep, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Workspace: the head words, the stage table, then the mirrors (each
// output's words 16-byte aligned).
static int64_t table_bytes(int nstages) { return (int64_t)kPassHeadWords * 4 + (int64_t)nstages * sizeof(PassStage); }

int64_t pass_workspace_bytes(int nstages, const int64_t *chained_rows, int nchained) {
    int64_t words = 0;
    for (int i = 0; i < nchained; i++) words += (chained_rows[i] + 1) & ~int64_t(1);
    return table_bytes(nstages) + 8 * words;
}

int pass_grid() {
    const int occ = occupancy(reinterpret_cast<const void *>(gemv_pass_kernel), kPassThreads,
                              (size_t)kPassLdsFloats * sizeof(float));
    // one workgroup per CU (more would stretch each stage's slowest row share)
    const int want = tuning(QK_TUNE_GEMV_WGS_PER_CU) > 0 ? tuning(QK_TUNE_GEMV_WGS_PER_CU) : 1;
    return device_cu_count() * (want < occ ? want : occ);
}

bool pass_stage_ok(int type, int64_t rows, int64_t cols) {
    if (type != Q4_K && type != Q6_K) return false;
    if (cols > kRegStageCols || rows < 1 || cols < 256) return false;
    if (!(type == Q4_K ? fast_ok<Q4_K>(rows, cols) : fast_ok<Q6_K>(rows, cols))) return false;
    return kPassCompute % make_plan<Q4_K>(cols).KS == 0;  // Q4_K and Q6_K share the plan
}

// The per-stage kernel's plan for this width (the same lanes per row and
// the same split, so the same bits), with the compute waves as row waves.
static GemvPlan pass_plan(int64_t cols) {
    GemvPlan p = make_plan<Q4_K>(cols);
    p.NWR = kPassCompute / p.KS;
    return p;
}

// Builds the stage table: items[first[s] .. first[s + 1]) are stage s (all of
// one width and one input, Q4_K/Q6_K, pass_stage_ok), G workgroups; ll_of[i]
// is the mirror word of items[i]'s y[0], or -1.
static int pass_table(const GemvItem *items, const int *first, int nstages, const int64_t *cols_of_stage,
                      const PassStageIn *in, const int64_t *ll_of, int G, std::vector<PassStage> &tab) {
    tab.assign((size_t)nstages, PassStage{});
    for (int s = 0; s < nstages; s++) {
        PassStage &st = tab[(size_t)s];
        std::memset(&st, 0, sizeof st);
        const int64_t cols = cols_of_stage[s];
        const GemvPlan p = pass_plan(cols);
        const int64_t RG = p.NWR * p.RP;
        // Q4_K matrices first (the format of matrices [0, n1)), then Q6_K
        int sorted[kGemvMaxMats];
        int n = 0, n1 = 0;
        for (int pass = 0; pass < 2; pass++)
            for (int i = first[s]; i < first[s + 1]; i++)
                if ((items[i].type == Q4_K) == (pass == 0)) sorted[n++] = i;
        for (int i = 0; i < n; i++) n1 += items[sorted[i]].type == Q4_K;
        GemvWork &w = st.w;
        const PassStageIn &pi = in[s];
        w.x = pi.x;
        w.in = GemvInput{0, nullptr, nullptr, 0.f, nullptr};
        w.W = static_cast<const uint8_t *>(items[sorted[0]].W);
        w.y = items[sorted[0]].y;
        st.kind = pi.kind;
        st.eps = pi.eps;
        st.x_ll = pi.x_src >= 0 ? ll_of[pi.x_src] : -1;
        st.aux_ll = pi.aux_src >= 0 ? ll_of[pi.aux_src] : -1;
        st.aux = pi.aux;
        st.norm_w = pi.norm_w;
        int64_t G_[kGemvMaxMats] = {0, 0, 0, 0};
        double bytes = 0.0;
        int64_t total = 0;
        for (int j = 0; j < kGemvMaxMats; j++) {
            const bool used = j < n;
            const GemvItem *it = used ? &items[sorted[j]] : nullptr;
            w.wof[j] = used ? (int64_t)((uintptr_t)it->W - (uintptr_t)w.W) : 0;
            w.yof[j] = used ? (int64_t)(((intptr_t)it->y - (intptr_t)w.y) / (intptr_t)sizeof(float)) : 0;
            w.rows[j] = used ? (int)it->rows : 1;
            st.y_ll[j] = used ? ll_of[sorted[j]] : -1;
            if (used) {
                G_[j] = (it->rows + RG - 1) / RG;
                total += G_[j];
            }
        }
        w.n1 = n1 > 0 ? n1 : n;
        const int f1 = n1 > 0 ? Q4_K : Q6_K, f2 = n1 < n ? Q6_K : f1;
        w.row_bytes[0] = (int)(cols / 256 * (f1 == Q4_K ? 144 : 210));
        w.row_bytes[1] = (int)(cols / 256 * (f2 == Q4_K ? 144 : 210));
        for (int j = 0; j < n; j++) bytes += (double)G_[j] * w.row_bytes[j < w.n1 ? 0 : 1];
        // workgroups per matrix: one per row group while they all fit, else in
        // proportion to the matrices' bytes (at least one each)
        int64_t wg[kGemvMaxMats] = {0, 0, 0, 0}, grid = 0;
        for (int j = 0; j < n; j++) {
            if (total <= G) {
                wg[j] = G_[j];
            } else {
                const double bj = (double)G_[j] * w.row_bytes[j < w.n1 ? 0 : 1];
                wg[j] = (int64_t)((double)G * bj / bytes);
                wg[j] = wg[j] < 1 ? 1 : (wg[j] > G_[j] ? G_[j] : wg[j]);
            }
            // every workgroup's rows (times KS partials) must fit the result buffer
            const int64_t mn = (G_[j] * RG * p.KS + kMaxRes - 1) / kMaxRes;
            if (wg[j] < mn) wg[j] = mn;
            grid += wg[j];
        }
        // proportional shares that round to more workgroups than the grid
        // holds are trimmed from the largest
        while (grid > G) {
            int jm = 0;
            for (int j = 1; j < n; j++)
                if (wg[j] > wg[jm]) jm = j;
            if (wg[jm] <= 1) return -1;
            wg[jm]--;
            grid--;
        }
        int64_t b = 0;
        for (int j = 0; j < kMaxMats; j++) {
            w.wgbeg[j] = (int)b;
            if (j < n) {
                if ((G_[j] + wg[j] - 1) / wg[j] * RG * p.KS > kMaxRes) return -1;
                w.q[j] = (int)(G_[j] / wg[j]);
                w.r[j] = (int)(G_[j] % wg[j]);
                b += wg[j];
            } else {
                w.q[j] = w.r[j] = 0;
            }
        }
        for (int j = n; j < kMaxMats; j++) w.wgbeg[j] = (int)b;
        st.p = p;
        st.f1 = f1;
        st.f2 = f2;
        st.split = p.KS > 1;
        st.wide = p.Lshift >= 4;
        st.nwg = (int)b;
    }
    return 0;
}

int pass_build(const GemvItem *items, int n, const int *first, int nstages, const int64_t *cols,
               const PassStageIn *in, const unsigned char *chained, int G, void *ws, hipError_t *herr) {
    // mirror words of the outputs that a later stage reads
    std::vector<int64_t> ll_of((size_t)n, -1);
    int64_t words = 0;
    for (int i = 0; i < n; i++) {
        if (!chained[i]) continue;
        ll_of[(size_t)i] = words;
        words += (items[i].rows + 1) & ~int64_t(1);  // 16-byte aligned
    }
    std::vector<PassStage> tab;
    if (pass_table(items, first, nstages, cols, in, ll_of.data(), G, tab) != 0) return -1;
    std::vector<uint8_t> img((size_t)table_bytes(nstages), 0);
    std::memcpy(img.data() + (size_t)kPassHeadWords * 4, tab.data(), tab.size() * sizeof(PassStage));
    *herr = hipMemcpy(ws, img.data(), img.size(), hipMemcpyHostToDevice);
    // mirror words of epoch 0, which no run takes as current
    if (*herr == hipSuccess && words > 0) *herr = hipMemset(static_cast<uint8_t *>(ws) + img.size(), 0, (size_t)(8 * words));
    if (*herr == hipSuccess) *herr = hipDeviceSynchronize();
    return *herr == hipSuccess ? 0 : -2;
}

hipError_t pass_launch(void *ws, int nstages, int G, int64_t limit, hipStream_t stream) {
    uint8_t *base = static_cast<uint8_t *>(ws);
    uint32_t *head = reinterpret_cast<uint32_t *>(base);
    const PassStage *tab = reinterpret_cast<const PassStage *>(base + (size_t)kPassHeadWords * 4);
    uint64_t *ll = reinterpret_cast<uint64_t *>(base + table_bytes(nstages));
    hipLaunchKernelGGL(gemv_pass_kernel, dim3((unsigned)G), dim3(kPassThreads), (size_t)kPassLdsFloats * sizeof(float),
                       stream, tab, nstages, head, ll, limit);
    return hipGetLastError();
}

hipError_t pass_last_error(const void *ws, uint32_t *err) {
    return hipMemcpy(err, static_cast<const uint8_t *>(ws) + kPassLastErr * 4, 4, hipMemcpyDeviceToHost);
}

static_assert(sizeof(PassStage) % 16 == 0, "stage table entries stay 16-byte aligned");
static_assert((kPassHeadWords * 4) % 16 == 0, "the stage table starts 16-byte aligned");

}  // namespace qk
