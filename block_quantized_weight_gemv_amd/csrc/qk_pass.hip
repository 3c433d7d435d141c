// qk_pass.hip — a whole decode-step weight pass in one persistent launch.
//
// The pages' forward pass runs the projections of a layer in a fixed order,
// each stage reading an x that the stage before produced ("picoLM, in
// Python", §4 — The forward pass: q, k and v read one normed x, o the
// attention output, gate and up another normed x, down the SwiGLU product).
// On this GPU a launch per stage costs more than the stage's own weight
// traffic at 1.1B shapes (an empty kernel in a graph takes ~1.7 us, a stage
// streams 3-11 MB in 1-2 us), so here one launch walks all the stages:
//
// * Every workgroup is resident (the grid is the occupancy times the CU
//   count) and walks the stage table in order. In stage s it takes its share
//   of the stage's row groups, exactly as a per-stage launch of the same
//   matrices would (gemv_body, the same plan and the same decode, so the
//   results are the same bits). A plan of 3 waves per row group lets the
//   fourth wave repeat the first one's rows.
// * Stage s may read an x written by stage s-1. A workgroup therefore
//   requests its first rows' weights, then waits until every workgroup has
//   finished stage s-1, then reads x: the weights are already on their way
//   while it waits. A workgroup with no rows in a stage does not wait.
// * Completion is counted per stage in eight counters (a workgroup adds to
//   the one of the XCD it runs on, so that the adds spread over eight cache
//   lines); a waiter reads the eight with one load instruction and compares
//   their sum with the grid size.
// * Visibility without cache flushes: y is written and x read with
//   device-scope (sc1) accesses, which are coherent across the XCDs' L2
//   caches, and a workgroup adds to its counter only after its y stores
//   have completed (s_waitcnt). A full release/acquire fence per workgroup
//   would write back and invalidate the L2 for every workgroup of every
//   stage.
// * Every wait is bounded: past a spin limit it sets an error word and goes
//   on (the results are then not to be trusted, but the launch ends). After
//   the last stage each workgroup counts itself out; the last one clears the
//   counters for the next run and records the error word.
#include <cstring>
#include <vector>

#include "qk_gemv_body.h"

namespace qk {

constexpr int kPassSlots = 8;         // counters per stage
constexpr int kPassSlotWords = 32;    // 128 bytes between counters
constexpr int kPassThreads = 256;     // 4 waves per workgroup

// The words at the start of the workspace.
enum { kPassErr = 0, kPassLastErr = 1, kPassExits = 2, kPassHeadWords = 32 };

struct PassStage {
    GemvWork w;  // the stage's matrices: x, W, y, offsets, rows, workgroup ranges
    GemvPlan p;
    int f1, f2;  // formats of matrices [0, n1) and [n1, n)
    int split;   // rows split over waves
    int wide;    // row slots of 16 or more lanes
    int nwg;     // workgroups with rows in this stage
    int pad[3];
};

struct PassSync {
    static constexpr bool kPersist = true;
    const uint32_t *cnt;  // the counters of the stage x comes from; nullptr: nothing to wait for
    uint32_t target;      // the grid size
    uint32_t *err;
    int64_t limit;        // polls before a wait gives up

    __device__ void wait() const {
        if (cnt != nullptr && threadIdx.x < 64) {
            const int lane = threadIdx.x;
            // (once a wait of this run has given up, later ones do not wait)
            if (__hip_atomic_load(err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
                for (int64_t it = 0;; it++) {
                    if (it >= limit) {  // a limit of 0 gives up at once
                        if (lane == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    uint32_t v = lane < kPassSlots ? __hip_atomic_load(cnt + lane * kPassSlotWords, __ATOMIC_RELAXED,
                                                                       __HIP_MEMORY_SCOPE_AGENT)
                                                   : 0u;
                    v += __shfl_xor(v, 1);
                    v += __shfl_xor(v, 2);
                    v += __shfl_xor(v, 4);
                    if (__builtin_amdgcn_readfirstlane(v) >= target) break;
                    __builtin_amdgcn_s_sleep(2);
                }
            }
        }
        __syncthreads();
    }
    __device__ float4 load_x(const float *p) const {
        return float4{__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                      __hip_atomic_load(p + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                      __hip_atomic_load(p + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                      __hip_atomic_load(p + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)};
    }
    __device__ void store_y(float *p, float v) const {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
};

template <int F, bool SPLIT, bool WIDE>
__device__ __forceinline__ void pass_gemv(const PassStage &st, const MatSel &ms, float *res, const PassSync &sync) {
    gemv_body<F, 2, SPLIT, WIDE, 0, 0, false, PassSync>(st.w.x, ms, res, st.w.in, sync);
}

template <int F>
__device__ __forceinline__ void pass_gemv_f(const PassStage &st, const MatSel &ms, float *res, const PassSync &sync,
                                            int split, int wide) {
    if (split) {
        if (wide)
            pass_gemv<F, true, true>(st, ms, res, sync);
        else
            pass_gemv<F, true, false>(st, ms, res, sync);
    } else {
        if (wide)
            pass_gemv<F, false, true>(st, ms, res, sync);
        else
            pass_gemv<F, false, false>(st, ms, res, sync);
    }
}

__global__ __launch_bounds__(kPassThreads) void gemv_pass_kernel(const PassStage *__restrict__ tab, int nstages,
                                                                 uint32_t *head, uint32_t *ctr, int64_t limit) {
    extern __shared__ __attribute__((aligned(16))) float res[];
    __shared__ uint32_t last;
    const uint32_t xcd = __builtin_amdgcn_s_getreg((3 << 11) | 20) & 7u;  // hwreg(HW_REG_XCC_ID, 0, 4)
    const int blk = (int)blockIdx.x;
    for (int s = 0; s < nstages; s++) {
        const PassStage &st = tab[s];
        if (blk < st.nwg) {
            const PassSync sync{s > 0 ? ctr + (int64_t)(s - 1) * kPassSlots * kPassSlotWords : nullptr, gridDim.x,
                                head + kPassErr, limit};
            const MatSel ms = mat_sel(st.w, st.p, blk);
            if ((ms.j == 0 ? st.f1 : st.f2) == Q4_K)
                pass_gemv_f<Q4_K>(st, ms, res, sync, st.split, st.wide);
            else
                pass_gemv_f<Q6_K>(st, ms, res, sync, st.split, st.wide);
        }
        // every y store of this workgroup is complete before it counts itself
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0)
            __hip_atomic_fetch_add(ctr + ((int64_t)s * kPassSlots + xcd) * kPassSlotWords, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
    // every counter add of this workgroup has landed before it counts itself
    // out; the last workgroup out clears the counters for the next run
    __builtin_amdgcn_s_waitcnt(0);
    if (threadIdx.x == 0)
        last = __hip_atomic_fetch_add(head + kPassExits, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
               gridDim.x - 1;
    __syncthreads();
    if (last) {
        for (int i = threadIdx.x; i < nstages * kPassSlots; i += blockDim.x)
            __hip_atomic_store(ctr + (int64_t)i * kPassSlotWords, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (threadIdx.x == 0) {
            const uint32_t e = __hip_atomic_load(head + kPassErr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(head + kPassLastErr, e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(head + kPassErr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(head + kPassExits, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// LDS of a pass workgroup: x (up to kRegStageCols columns, padded) and its
// sums, then the split rows' partial results.
constexpr int64_t kPassLdsFloats = 6528 + 384 + kMaxRes;
static_assert(kPassLdsFloats >= ((kRegStageCols + 4 * (kRegStageCols / 64) + kRegStageCols / 16 + 3) & ~3) + kMaxRes,
              "pass LDS holds the widest x and the partial results");

int64_t pass_workspace_bytes(int nstages) {
    return (int64_t)kPassHeadWords * 4 + (int64_t)nstages * kPassSlots * kPassSlotWords * 4 +
           (int64_t)nstages * (int64_t)sizeof(PassStage);
}

int pass_grid() {
    const int occ = occupancy(reinterpret_cast<const void *>(gemv_pass_kernel), kPassThreads,
                              (size_t)kPassLdsFloats * sizeof(float));
    // one workgroup per CU: every stage's barrier costs more with more
    // workgroups (1.1B decode pass: 6.3 us per stage with 256, 8.3 with 512)
    const int want = tuning(QK_TUNE_GEMV_WGS_PER_CU) > 0 ? tuning(QK_TUNE_GEMV_WGS_PER_CU) : 1;
    return device_cu_count() * (want < occ ? want : occ);
}

bool pass_stage_ok(int type, int64_t rows, int64_t cols) {
    if (type != Q4_K && type != Q6_K) return false;
    if (cols > kRegStageCols || rows < 1 || cols < 256) return false;
    if (!(type == Q4_K ? fast_ok<Q4_K>(rows, cols) : fast_ok<Q6_K>(rows, cols))) return false;
    const GemvPlan p = make_plan<Q4_K>(cols);  // Q4_K and Q6_K share the plan
    return p.KS * p.NWR <= 4;
}

// Builds the stage table: items[first[s] .. first[s + 1]) are stage s (all of
// one width and one x, Q4_K/Q6_K, pass_stage_ok), G workgroups.
static int pass_table(const GemvItem *items, const int *first, int nstages, const int64_t *cols_of_stage,
                      const float *const *x_of_stage, int G, std::vector<PassStage> &tab) {
    tab.assign((size_t)nstages, PassStage{});
    for (int s = 0; s < nstages; s++) {
        PassStage &st = tab[(size_t)s];
        std::memset(&st, 0, sizeof st);
        const int64_t cols = cols_of_stage[s];
        const GemvPlan p = make_plan<Q4_K>(cols);
        const int64_t RG = p.NWR * p.RP;
        // Q4_K matrices first (the format of matrices [0, n1)), then Q6_K
        GemvItem sorted[kGemvMaxMats];
        int n = 0, n1 = 0;
        for (int pass = 0; pass < 2; pass++)
            for (int i = first[s]; i < first[s + 1]; i++)
                if ((items[i].type == Q4_K) == (pass == 0)) sorted[n++] = items[i];
        for (int i = 0; i < n; i++) n1 += sorted[i].type == Q4_K;
        GemvWork &w = st.w;
        w.x = x_of_stage[s];
        w.in = GemvInput{0, nullptr, nullptr, 0.f, nullptr};
        w.W = static_cast<const uint8_t *>(sorted[0].W);
        w.y = sorted[0].y;
        int64_t G_[kGemvMaxMats] = {0, 0, 0, 0};
        double bytes = 0.0;
        int64_t total = 0;
        for (int j = 0; j < kGemvMaxMats; j++) {
            const bool used = j < n;
            w.wof[j] = used ? (int64_t)((uintptr_t)sorted[j].W - (uintptr_t)sorted[0].W) : 0;
            w.yof[j] = used ? (int64_t)(((intptr_t)sorted[j].y - (intptr_t)sorted[0].y) / (intptr_t)sizeof(float)) : 0;
            w.rows[j] = used ? (int)sorted[j].rows : 1;
            if (used) {
                G_[j] = (sorted[j].rows + RG - 1) / RG;
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
            if (p.KS > 1) {
                // every workgroup's rows (times KS partials) must fit the result buffer
                const int64_t mn = (G_[j] * RG * p.KS + kMaxRes - 1) / kMaxRes;
                if (wg[j] < mn) wg[j] = mn;
            }
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
                if (p.KS > 1 && (G_[j] + wg[j] - 1) / wg[j] * RG * p.KS > kMaxRes) return -1;
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

int pass_build(const GemvItem *items, const int *first, int nstages, const int64_t *cols, const float *const *xs,
               int G, void *ws, hipError_t *herr) {
    std::vector<PassStage> tab;
    if (pass_table(items, first, nstages, cols, xs, G, tab) != 0) return -1;
    std::vector<uint8_t> img((size_t)pass_workspace_bytes(nstages), 0);
    std::memcpy(img.data() + (size_t)kPassHeadWords * 4 + (size_t)nstages * kPassSlots * kPassSlotWords * 4,
                tab.data(), tab.size() * sizeof(PassStage));
    *herr = hipMemcpy(ws, img.data(), img.size(), hipMemcpyHostToDevice);
    return *herr == hipSuccess ? 0 : -2;
}

hipError_t pass_launch(void *ws, int nstages, int G, int64_t limit, hipStream_t stream) {
    uint8_t *base = static_cast<uint8_t *>(ws);
    uint32_t *head = reinterpret_cast<uint32_t *>(base);
    uint32_t *ctr = head + kPassHeadWords;
    const PassStage *tab = reinterpret_cast<const PassStage *>(base + (size_t)kPassHeadWords * 4 +
                                                               (size_t)nstages * kPassSlots * kPassSlotWords * 4);
    hipLaunchKernelGGL(gemv_pass_kernel, dim3((unsigned)G), dim3(kPassThreads), (size_t)kPassLdsFloats * sizeof(float),
                       stream, tab, nstages, head, ctr, limit);
    return hipGetLastError();
}

hipError_t pass_last_error(const void *ws, uint32_t *err) {
    return hipMemcpy(err, static_cast<const uint8_t *>(ws) + kPassLastErr * 4, 4, hipMemcpyDeviceToHost);
}

static_assert(sizeof(PassStage) % 16 == 0, "stage table entries stay 16-byte aligned");

}  // namespace qk
