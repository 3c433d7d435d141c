// qk_launch.h — host-side launchers behind the C ABI (qk_api.cpp).
// Arguments reaching these have already been validated by the API layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qk.h"

namespace qk {

// Compute units of the current device (cached per device).
int device_cu_count();
// LDS bytes one workgroup may allocate on the current device (cached per
// device; 160 KiB on gfx950).
int device_lds_per_block();
// Lets kern use the device's whole per-workgroup LDS (less its static LDS) as
// dynamic LDS; recorded per device and kernel, so that each device is set
// once. Returns the HIP error of the attribute calls.
hipError_t allow_max_dynamic_lds(const void *kern);

// Sets the calling thread's qk_last_error() message (a copy of msg); returns status.
int set_last_error(int status, const char *msg);

// Workgroups of `kern` resident per CU at this block size and dynamic LDS on
// the current device (cached per device, kernel and configuration; 1 if the
// runtime gives no answer).
int occupancy(const void *kern, int threads, size_t lds_bytes);

// The value set for a tuning key (qk_set_tuning, QK_TUNE_*), or -1 for the
// dispatch table's own choice.
int tuning(int key);

hipError_t launch_dequant(int type, const void *blocks, int64_t n, float *out, hipStream_t stream);

hipError_t launch_gemv(int type, const void *W, int64_t rows, int64_t cols, const float *x, float *y,
                       hipStream_t stream);

// GEMVs of one width against one x in one launch. Formats with the same
// unit layout (Q4_K with Q6_K, q4_0 with q8_0) may be mixed.
constexpr int kGemvMaxMats = 4;
struct GemvItem {
    int type;
    const void *W;
    int64_t rows;
    float *y;
};
// Whether the fused kernel takes this format and shape.
bool gemv_fusable(int type, int64_t rows, int64_t cols);
// Whether GEMVs of formats a and b may share one launch.
bool gemv_groupable(int a, int b);
// A transform of x applied as it is staged: kind 0 none; 1 x' = RMSNorm(x +
// aux) * norm_w (eps), x + aux also written to x_out; 2 x' = silu(x) * aux.
struct GemvInput {
    int kind;
    const float *aux;
    const float *norm_w;
    float eps;
    float *x_out;
};
// Whether a transformed input is available for this format and shape.
bool gemv_input_ok(int type, int64_t rows, int64_t cols);
// The kernel a single GEMV of this format and shape runs: 0 generic, 1 fused
// (rows read straight into registers), 2 fused with rows streamed through
// LDS, 3 the wide-row kernel.
int gemv_path(int type, int64_t rows, int64_t cols);
// 1 <= n <= kGemvMaxMats items, all gemv_fusable, pairwise groupable; xin
// NULL or kind 0 for plain x (else every item gemv_input_ok).
hipError_t launch_gemv_group(const GemvItem *items, int n, int64_t cols, const float *x, hipStream_t stream,
                             const GemvInput *xin = nullptr);

// The persistent decode pass (qk_pass.hip).
// A stage's input: x, and for SwiGLU aux, each either read from memory or
// the output of an earlier GEMV of the pass (then read from that output's
// mirror); the transform applied to it (0 none, 1 RMSNorm with optional
// weights, 2 silu(x) * aux).
struct PassStageIn {
    int kind;
    const float *x;
    int x_src;  // index of the GEMV whose output x is, or -1
    const float *aux;
    int aux_src;
    const float *norm_w;
    float eps;
};
// Workspace bytes of a pass of nstages stages whose chained outputs (read by
// a later stage) have the given row counts.
int64_t pass_workspace_bytes(int nstages, const int64_t *chained_rows, int nchained);
// Workgroups of a pass launch on the current device (all resident).
int pass_grid();
// Whether a GEMV of this format and shape can be a pass stage member.
bool pass_stage_ok(int type, int64_t rows, int64_t cols);
// Builds the stage table of a pass for G workgroups — items[first[s] ..
// first[s + 1]) are stage s, of width cols[s] and input in[s]; chained[i]
// says that a later stage reads items[i]'s output — and copies it into ws,
// with the head words and the mirrors zeroed (blocking). Returns 0, -1 when
// a stage's rows do not fit the plan, or -2 with *herr set on a HIP error.
int pass_build(const GemvItem *items, int n, const int *first, int nstages, const int64_t *cols,
               const PassStageIn *in, const unsigned char *chained, int G, void *ws, hipError_t *herr);
hipError_t pass_launch(void *ws, int nstages, int G, int64_t limit, hipStream_t stream);
hipError_t pass_last_error(const void *ws, uint32_t *err);

hipError_t launch_gemm(int type, const void *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M,
                       float *Y, hipStream_t stream);

hipError_t launch_fill_zero(float *p, int64_t n, hipStream_t stream);

}  // namespace qk
