// qk_gemm.hip — Y = X W^T for M activation rows (bf16 X, fp32 Y).
//
// The multi-token path ("picoLM, in Python" prefills one position at a time;
// batching positions turns the GEMV into a dense contraction):
// * gemm_few_kernel (1 < M <= 16, K-quants): W streams once through the
//   MFMA, codes exact in bf16, scales applied per group in fp32;
// * gemm_prefill_kernel (M > 16, K-quants): X tiles in LDS, each wave decodes
//   its weight rows into exact bf16 hi/lo operands (two MFMAs per product);
// * gemm_rows_kernel (the 32-weight formats and the ggml formats): one wave
//   per weight row; lanes walk the row four weights at a time with the bit-exact decoder
//   and accumulate up to MB activation rows at once, so W is streamed once per
//   MB rows of X.
#include "qk_decode.h"
#include "qk_launch.h"

namespace qk {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __builtin_bit_cast(float, v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __builtin_bit_cast(float, v & 0xFFFF0000u); }

template <int F, int MB>
__global__ __launch_bounds__(256) void gemm_rows_kernel(const uint8_t *__restrict__ W, int64_t rows, int64_t cols,
                                                        int64_t row_bytes, const uint16_t *__restrict__ X,
                                                        int64_t M, float *__restrict__ Y) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    const int lane = threadIdx.x & 63;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x >> 6);
    const int64_t mchunks = (M + MB - 1) / MB;
    for (int64_t job = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); job < rows * mchunks;
         job += nwaves) {
        const int64_t r = job % rows, m0 = (job / rows) * MB;
        const uint8_t *row = W + r * row_bytes;
        float acc[MB];
#pragma unroll
        for (int m = 0; m < MB; m++) acc[m] = 0.f;
        for (int64_t c = 4 * (int64_t)lane; c < cols; c += 256) {
            float w[4];
            decode4<F>(row + (c / QK) * BYTES, (int)(c % QK), w);
#pragma unroll
            for (int m = 0; m < MB; m++) {
                if (m0 + m < M) {
                    const uint2 xv = *reinterpret_cast<const uint2 *>(X + (m0 + m) * cols + c);
                    acc[m] += w[0] * bf16_lo(xv.x) + w[1] * bf16_hi(xv.x) + w[2] * bf16_lo(xv.y) +
                              w[3] * bf16_hi(xv.y);
                }
            }
        }
#pragma unroll
        for (int m = 0; m < MB; m++) {
            float a = acc[m];
            for (int s = 32; s > 0; s >>= 1) a += __shfl_xor(a, s);
            if (lane == 0 && m0 + m < M) Y[(m0 + m) * rows + r] = a;
        }
    }
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Two fp32 values whose low 16 bits are zero (or to be dropped) as a bf16 pair.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
}

// ---------------------------------------------------------------------------
// Few-token kernel (M <= 16, K-quants): the same exact-code MFMA scheme
// with W read straight from global memory, laid out like the GEMV so that W
// streams once; only X passes through LDS.
//
// A wave owns 16 weight rows (the MFMA's N) and a range of super-blocks; the
// KSW waves of a workgroup split the row's super-blocks and add their 16 x 16
// partial tiles in LDS. Lane l holds the B operand for weight row l % 16,
// read straight from global memory, and the A operand for token l % 16 from
// the wave's X tile, both at k-chunk l / 16; the next super-block's loads are
// in flight while one is multiplied. A nibble or 6-bit code c becomes the bf16 value 128 + c
// with one v_perm_b32 per two codes (bits 0x43cc); a second MFMA against ones
// gives the sum of X over the group, and the group's scale removes the
// offset:  Q4_K  acc += d*sc*P - (128*d*sc + dmin*min)*S
//          Q6_K  acc += d*sc*(P - 160*S)   (offset 128 plus the code's -32)
// so no weight is ever rounded.
// ---------------------------------------------------------------------------

// bf16 pairs (128 + b0, 128 + b1) and (128 + b2, 128 + b3) of the four bytes of v
__device__ __forceinline__ uint32_t bf16_off_lo(uint32_t v) { return __builtin_amdgcn_perm(0x43434343u, v, 0x04010400u); }
__device__ __forceinline__ uint32_t bf16_off_hi(uint32_t v) { return __builtin_amdgcn_perm(0x43434343u, v, 0x04030402u); }

template <int F> struct FewRaw;
template <> struct FewRaw<Q4_K> {
    u32x4 h;      // d | dmin | packed scales and mins
    u32x2 q[4];   // nibble bytes 32g + 8c .. +7 of the four nibble groups
};
template <> struct FewRaw<Q6_K> {
    u32x2 a[4], b[4], qh[4];  // per (h, lh): ql, ql + 32, qh windows (aligned down)
    u32x4 s;                  // scales (window)
    uint32_t s4;              // q6k_tail: scales 14, 15 and d
};

// X reaches the MFMA through a wave-private LDS tile of 16 token rows x 256
// columns (one super-block; rows padded by 16 bytes): lane l loads 16-byte
// chunk l % 32 of token rows l / 32, 2 + l / 32, ... (coalesced along the
// row; rows past M load row M - 1 again, whose products are never stored),
// stores them to the tile, and reads its A operands (token l % 16) from it.
// Read straight from X by each lane for its own token, the 16 token rows of
// one load instruction sit ldx apart (4 KiB at 2048 columns) and fall on the
// same L1 cache sets; the tag conflicts stalled the address pipeline.
constexpr int FEW_LX = 264;  // bf16 per tile row
// NP (1, 2, 4 or 8) pairs of token rows are loaded, the fewest that cover
// M: tile rows past them are never written, and the garbage the MFMA then
// reads there only reaches result rows of tokens past M, which are not stored.
template <int NP>
struct FewX {
    u32x4 v[NP];
};
template <int NP>
__device__ __forceinline__ void few_xload(FewX<NP> &x, const uint16_t *X, int64_t ldx, int kb, int M, int lane) {
#pragma unroll
    for (int i = 0; i < NP; i++) {
        const int row = min(2 * i + (lane >> 5), M - 1);
        x.v[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)row * ldx + (int64_t)kb * 256 + 8 * (lane & 31));
    }
}
template <int NP>
__device__ __forceinline__ void few_xstore(const FewX<NP> &x, uint16_t *xw, int lane) {
#pragma unroll
    for (int i = 0; i < NP; i++)
        *reinterpret_cast<u32x4 *>(xw + (2 * i + (lane >> 5)) * FEW_LX + 8 * (lane & 31)) = x.v[i];
}

template <int F>
__device__ __forceinline__ void few_load(FewRaw<F> &r, const uint8_t *blk, int c);

template <>
__device__ __forceinline__ void few_load<Q4_K>(FewRaw<Q4_K> &r, const uint8_t *blk, int c) {
    r.h = ld_b128(blk);
#pragma unroll
    for (int g = 0; g < 4; g++) r.q[g] = ld_b64(blk + 16 + 32 * g + 8 * c);
}

template <>
__device__ __forceinline__ void few_load<Q6_K>(FewRaw<Q6_K> &r, const uint8_t *blk, int c) {
    const uint8_t *A0 = blk - ((uintptr_t)blk & 3u);  // 4-byte aligned base; blk is 2-byte aligned
#pragma unroll
    for (int hl = 0; hl < 4; hl++) {
        const int h = hl >> 1, lh = hl & 1;
        r.a[hl] = ld_b64(A0 + 64 * h + 16 * lh + 4 * c);
        r.b[hl] = ld_b64(A0 + 64 * h + 32 + 16 * lh + 4 * c);
        r.qh[hl] = ld_b64(A0 + 128 + 32 * h + 16 * lh + 4 * c);
    }
    r.s = ld_b128(A0 + 192);
    r.s4 = q6k_tail(blk);
}

// xa: this lane's token row of the X tile (token n = lane % 16), offset to
// its k chunk c = lane / 16 (8 columns of the chunk for Q4_K, 4 for Q6_K).
template <int F>
__device__ __forceinline__ void few_mma(const FewRaw<F> &r, const uint8_t *blk, const uint16_t *xa, f32x4 &acc);

template <>
__device__ __forceinline__ void few_mma<Q4_K>(const FewRaw<Q4_K> &r, const uint8_t *, const uint16_t *xa,
                                              f32x4 &acc) {
    const u32x4 h = r.h;
    const float d = half_bits_to_float(h.x & 0xFFFFu), dmin = half_bits_to_float(h.x >> 16);
    const uint32_t sc_lo = h.y & 0x3F3F3F3Fu, mn_lo = h.z & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t mn_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    const u32x4 ones = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t SC = j < 4 ? sc_lo : sc_hi, MN = j < 4 ? mn_lo : mn_hi;
        const float dsc = d * (float)((SC >> (8 * (j & 3))) & 0xFFu);
        const float dmn = dmin * (float)((MN >> (8 * (j & 3))) & 0xFFu);
        const u32x2 q = r.q[j >> 1];
        const uint32_t n0 = (j & 1) ? (q.x >> 4) & 0x0F0F0F0Fu : q.x & 0x0F0F0F0Fu;
        const uint32_t n1 = (j & 1) ? (q.y >> 4) & 0x0F0F0F0Fu : q.y & 0x0F0F0F0Fu;
        const u32x4 bw = u32x4{bf16_off_lo(n0), bf16_off_hi(n0), bf16_off_lo(n1), bf16_off_hi(n1)};
        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(xa + 32 * j);  // X[t][32j + 8c .. +7]
        const f32x4 P = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, bw),
                                                               f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const f32x4 S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, __builtin_bit_cast(bf16x8, ones),
                                                               f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float cj = 128.f * dsc + dmn;
        acc += dsc * P;
        acc -= cj * S;
    }
}

template <>
__device__ __forceinline__ void few_mma<Q6_K>(const FewRaw<Q6_K> &r, const uint8_t *blk, const uint16_t *xa,
                                              f32x4 &acc) {
    const uint32_t mis = (uint32_t)(uintptr_t)blk & 3u;
    const uint32_t s0 = align_bytes(r.s.y, r.s.x, mis), s1 = align_bytes(r.s.z, r.s.y, mis);
    const uint32_t s2 = align_bytes(r.s.w, r.s.z, mis), s3 = align_bytes(r.s4, r.s.w, mis);
    const uint32_t sw[4] = {s0, s1, s2, s3};  // scales 0..15
    const float d = half_bits_to_float(r.s4 >> 16);
    const u32x2 ones = u32x2{0x3F803F80u, 0x3F803F80u};
#pragma unroll
    for (int hl = 0; hl < 4; hl++) {
        const int h = hl >> 1, lh = hl & 1;
        const uint32_t A = align_bytes(r.a[hl].y, r.a[hl].x, mis);
        const uint32_t B = align_bytes(r.b[hl].y, r.b[hl].x, mis);
        const uint32_t H = align_bytes(r.qh[hl].y, r.qh[hl].x, mis);
        const uint32_t code[4] = {(A & 0x0F0F0F0Fu) | ((H << 4) & 0x30303030u),
                                  (B & 0x0F0F0F0Fu) | ((H << 2) & 0x30303030u),
                                  ((A >> 4) & 0x0F0F0F0Fu) | (H & 0x30303030u),
                                  ((B >> 4) & 0x0F0F0F0Fu) | ((H >> 2) & 0x30303030u)};
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int gi = 8 * h + 2 * k + lh;
            const float dsc = d * (float)(int)(int8_t)(sw[gi >> 2] >> (8 * (gi & 3)));
            const u32x2 bw = u32x2{bf16_off_lo(code[k]), bf16_off_hi(code[k])};
            const s16x4 av = *reinterpret_cast<const s16x4 *>(xa + 16 * gi);  // X[t][16 gi + 4c .. +3]
            const f32x4 P = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, bw),
                                                                     f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            const f32x4 S = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, __builtin_bit_cast(s16x4, ones),
                                                                     f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            acc += dsc * (P - 160.f * S);
        }
    }
}

template <int F, int NP>
__global__ __launch_bounds__(512) void gemm_few_kernel(const uint8_t *__restrict__ W, int rows, int nb,
                                                       int64_t row_bytes, const uint16_t *__restrict__ X, int M,
                                                       float *__restrict__ Y) {
    constexpr int BYTES = Layout<F>::BYTES;
    __shared__ f32x4 part[8][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ksw = blockDim.x >> 6;
    const int n = lane & 15, c = lane >> 4;
    const int r = min((int)blockIdx.x * 16 + n, rows - 1);
    const uint8_t *wrow = W + (int64_t)r * row_bytes;
    const int64_t ldx = (int64_t)nb * 256;
    extern __shared__ __attribute__((aligned(16))) uint16_t few_xs[];
    uint16_t *const xw = few_xs + wave * 16 * FEW_LX;   // this wave's X tile
    // its A operands: k chunk c is 8 columns wide for the 16x16x32 product
    // (Q4_K), 4 for the 16x16x16 one (Q6_K)
    const uint16_t *const xa = xw + n * FEW_LX + (F == Q4_K ? 8 : 4) * c;
    // this workgroup's share of the super-blocks (all of them, or one of two
    // halves), and this wave's part of it [kb0, kb1), spread evenly
    const int h0 = (int)blockIdx.y * nb / (int)gridDim.y, hn = ((int)blockIdx.y + 1) * nb / (int)gridDim.y - h0;
    const int kb0 = h0 + wave * hn / ksw, kb1 = h0 + (wave + 1) * hn / ksw;

    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    FewRaw<F> buf[2];
    FewX<NP> xn;
    // (every wave has at least one super-block: the host keeps ksw <= nb)
    few_xload(xn, X, ldx, kb0, M, lane);
    few_load<F>(buf[0], wrow + (int64_t)kb0 * BYTES, c);
    few_xstore(xn, xw, lane);
    for (int kb = kb0; kb < kb1; kb += 2) {
        // the next super-block's X and W loads go out before this one is
        // multiplied, and its X tile replaces this one's after the
        // multiplies (LDS accesses of a wave stay in order); loads are
        // unconditional (clamped to the wave's last super-block): a load
        // under a branch would make the compiler wait for all of them
        const int k1 = min(kb + 1, kb1 - 1);
        few_xload(xn, X, ldx, k1, M, lane);
        few_load<F>(buf[1], wrow + (int64_t)k1 * BYTES, c);
        __builtin_amdgcn_sched_barrier(0);
        few_mma<F>(buf[0], wrow + (int64_t)kb * BYTES, xa, acc);
        few_xstore(xn, xw, lane);
        const int k2 = min(kb + 2, kb1 - 1);
        few_xload(xn, X, ldx, k2, M, lane);
        few_load<F>(buf[0], wrow + (int64_t)k2 * BYTES, c);
        __builtin_amdgcn_sched_barrier(0);
        if (kb + 1 < kb1) few_mma<F>(buf[1], wrow + (int64_t)k1 * BYTES, xa, acc);
        few_xstore(xn, xw, lane);
    }
    // add the KSW partial tiles in a fixed order; lane holds tokens 4c+i of row n
    part[wave][lane] = acc;
    __syncthreads();
    if (wave == 0) {
        f32x4 t = part[0][lane];
        for (int w = 1; w < ksw; w++) t += part[w][lane];
        const int row = (int)blockIdx.x * 16 + n;
        if (row < rows) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int m = 4 * c + i;
                if (m >= M) continue;
                // two halves: each adds its sum to the zeroed output; with
                // exactly two addends the result does not depend on their order
                if (gridDim.y == 1)
                    Y[(int64_t)m * rows + row] = t[i];
                else
                    atomicAdd(&Y[(int64_t)m * rows + row], t[i]);
            }
        }
    }
}


template <int F, int NP>
static hipError_t launch_few_np(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                             int64_t M, float *Y, hipStream_t stream) {
    const int nb = (int)(cols / 256);
    const int64_t tiles = (rows + 15) / 16;
    // Row tiles that leave half the CUs or more without a workgroup, with at
    // least 16 super-blocks per row, are split over two workgroups, each over
    // half the super-blocks, which add their sums into the output zeroed by a
    // launch before (2048 x 5632 Q6_K: 12-17 % faster at M = 2-16; rows of 3
    // and 8 super-blocks were slower, the zeroing launch costing more than
    // the split gains). QK_TUNE_FEW_KH = 1/2 forces it.
    const int64_t cus = device_cu_count();
    const int kh_force = tuning(QK_TUNE_FEW_KH);
    int kh = kh_force > 0 ? kh_force : (tiles * 2 <= cus && nb >= 16 ? 2 : 1);
    if (kh != 2 || nb < 2) kh = 1;
    // about 4 waves per CU and at most 4 per workgroup (swept over 1, 2, 4 and
    // 8 waves per row tile at M = 2, 8, 16 on matrices of 2048 to 32000 rows
    // and 2048 to 14336 columns: fewer waves leave the memory pipes idle, more
    // split the row's super-blocks too finely); no more than one wave per
    // super-block
    const int64_t wgs = tiles * kh;
    int64_t ksw = (cus * 4 + wgs - 1) / wgs;
    if (ksw > 4) ksw = 4;
    if (tuning(QK_TUNE_FEW_KSW) > 0) ksw = tuning(QK_TUNE_FEW_KSW);  // waves per workgroup
    if (ksw > 8) ksw = 8;
    if (ksw > nb / kh) ksw = nb / kh;
    if (ksw < 1) ksw = 1;
    const size_t shmem = (size_t)ksw * 16 * FEW_LX * sizeof(uint16_t);  // the waves' X tiles
    if (shmem > 49152) {
        // more than the default dynamic LDS (set once per device)
        const hipError_t e = allow_max_dynamic_lds(reinterpret_cast<const void *>(gemm_few_kernel<F, NP>));
        if (e != hipSuccess) return e;
    }
    if (kh == 2) {
        const hipError_t ez = launch_fill_zero(Y, M * rows, stream);
        if (ez != hipSuccess) return ez;
    }
    hipLaunchKernelGGL((gemm_few_kernel<F, NP>), dim3((unsigned)tiles, (unsigned)kh), dim3((unsigned)(64 * ksw)), shmem,
                       stream, W, (int)rows, nb, row_bytes, X, (int)M, Y);
    return hipGetLastError();
}

template <int F>
static hipError_t launch_few(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                             int64_t M, float *Y, hipStream_t stream) {
    if (M <= 2) return launch_few_np<F, 1>(W, rows, cols, row_bytes, X, M, Y, stream);
    if (M <= 4) return launch_few_np<F, 2>(W, rows, cols, row_bytes, X, M, Y, stream);
    if (M <= 8) return launch_few_np<F, 4>(W, rows, cols, row_bytes, X, M, Y, stream);
    return launch_few_np<F, 8>(W, rows, cols, row_bytes, X, M, Y, stream);
}

// ---------------------------------------------------------------------------
// Prefill kernel (M > 16, K-quants): X tiles double-buffered in LDS, weights
// decoded straight into MFMA operands, scales folded into the operands.
//
// A workgroup computes 64 tokens x 64 weight rows; each of its 4 waves owns
// 16 rows and all 64 tokens (4 M tiles). Per K step of one
// super-block: the 64 x 256 X tile sits in LDS (shared by the 4 waves), the
// wave's weight rows are decoded in registers (lane l: row l % 16, k chunk
// l / 16), and the next step's X tile and weights are loaded while this one
// is multiplied; one barrier per step.
//
// Each v_mfma_f32_16x16x32_bf16 covers 32 columns. Its B operand is the
// integer v = scale * code of each weight, exact in fp32: Q4_K sc*q (at most
// 945, 10 significant bits), Q6_K sc*(q - 32) with sc in [-128, 127] and
// q - 32 in [-32, 31] (|v| <= 4096, 13 significant bits). bf16 holds 8
// significant bits, so v is split exactly into v_hi (v with the low 16 bits
// of its fp32 pattern cleared) and v_lo = v - v_hi (at most 5 significant
// bits), and two MFMAs accumulate X*v_hi + X*v_lo in fp32: every product is
// exact, only the fp32 accumulation rounds. The super-block's d multiplies
// the accumulated result once. Q4_K's minimum term, sum_j mn_j * (sum of X
// over sub-block j), is a third MFMA with B = mn_j (6 bits, exact) whose
// result dmin multiplies. No per-group scaling runs on the VALU.
// ---------------------------------------------------------------------------

constexpr int PF_TM = 64;     // tokens per workgroup
constexpr int PF_LROW = 264;  // LDS row pitch of the X tile (bf16): 256 + 8

template <int F> struct PfRaw;
template <> struct PfRaw<Q4_K> {
    u32x4 h;      // d | dmin | packed scales and mins
    u32x2 q[4];   // nibble bytes 32g + 8c .. +7 of the four nibble groups
};
template <> struct PfRaw<Q6_K> {
    u32x4 ql[4];  // ql bytes 64h + 32p + 8c .. (+ realignment) for (h, p)
    u32x4 qh[2];  // qh bytes 32h + 8c ..
    u32x4 s;      // scales (window)
    uint32_t s4;  // q6k_tail: scales 14, 15 and d
    uint32_t mis; // bytes from the 4-byte boundary below the block to it (0 or 2)
};

__device__ __forceinline__ void pf_load(PfRaw<Q4_K> &r, const uint8_t *blk, int c) {
    r.h = ld_b128(blk);
#pragma unroll
    for (int g = 0; g < 4; g++) r.q[g] = ld_b64(blk + 16 + 32 * g + 8 * c);
}

__device__ __forceinline__ void pf_load(PfRaw<Q6_K> &r, const uint8_t *blk, int c) {
    r.mis = (uint32_t)(uintptr_t)blk & 3u;
    const uint8_t *A0 = blk - r.mis;  // 4-byte aligned; every window below stays inside the block pair
#pragma unroll
    for (int hp = 0; hp < 4; hp++) r.ql[hp] = ld_b128(A0 + 64 * (hp >> 1) + 32 * (hp & 1) + 8 * c);
#pragma unroll
    for (int h = 0; h < 2; h++) r.qh[h] = ld_b128(A0 + 128 + 32 * h + 8 * c);
    r.s = ld_b128(A0 + 192);
    r.s4 = q6k_tail(blk);
}

// The exact split of eight fp32 integers v into bf16 operands: hi keeps the
// top 16 bits of each fp32 pattern (8 significant bits), lo = v - hi is
// exact with the few bits left, so both pack to bf16 by truncation.
__device__ __forceinline__ void split8(const float v[8], u32x4 &bh, u32x4 &bl) {
    float hi[8], lo[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        hi[e] = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, v[e]) & 0xFFFF0000u);
        lo[e] = v[e] - hi[e];
    }
    bh = u32x4{pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3]), pack_bf16(hi[4], hi[5]), pack_bf16(hi[6], hi[7])};
    bl = u32x4{pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3]), pack_bf16(lo[4], lo[5]), pack_bf16(lo[6], lo[7])};
}

// The A operands (X) of one 32-column chunk for the 4 M tiles, from LDS.
__device__ __forceinline__ void pf_xa(const uint16_t *xt, int lane, int k0, bf16x8 (&av)[4]) {
    const int c = lane >> 4;
#pragma unroll
    for (int a = 0; a < 4; a++)
        av[a] = *reinterpret_cast<const bf16x8 *>(xt + (16 * a + (lane & 15)) * PF_LROW + k0 + 8 * c);
}

// One 32-column chunk for the 4 M tiles: ah[a] += X_a * v_hi, al[a] += X_a *
// v_lo (separate accumulators, so consecutive MFMAs do not wait on each
// other) and, with MIN, am[a] += X_a * bm.
template <bool MIN>
__device__ __forceinline__ void pf_chunk(const bf16x8 (&av)[4], const u32x4 &bh, const u32x4 &bl, const u32x4 &bm,
                                         f32x4 (&ah)[4], f32x4 (&al)[4], f32x4 (&am)[4]) {
#pragma unroll
    for (int a = 0; a < 4; a++) {
        ah[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bh), ah[a], 0, 0, 0);
        al[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bl), al[a], 0, 0, 0);
        if constexpr (MIN)
            am[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bm), am[a], 0, 0, 0);
    }
}

// B operands of one 32-column chunk: the exact split v_hi + v_lo of the
// scaled codes (and, for Q4_K, the sub-block's minimum).
struct PfB {
    u32x4 h, l, m;
};

struct PfScalesQ4K {
    uint32_t sc_lo, mn_lo, sc_hi, mn_hi;
};

__device__ __forceinline__ PfScalesQ4K pf_scales(const PfRaw<Q4_K> &r) {
    const u32x4 h = r.h;
    return PfScalesQ4K{h.y & 0x3F3F3F3Fu, h.z & 0x3F3F3F3Fu, (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u),
                       ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u)};
}

// Q4_K sub-block j: v = sc * n (n the nibble), split exactly; B = mn for the minimum.
__device__ __forceinline__ PfB pf_dec(const PfRaw<Q4_K> &r, const PfScalesQ4K &S, int j) {
    const uint32_t SC = j < 4 ? S.sc_lo : S.sc_hi, MN = j < 4 ? S.mn_lo : S.mn_hi;
    const float sc = (float)((SC >> (8 * (j & 3))) & 0xFFu);
    const uint32_t mn = (MN >> (8 * (j & 3))) & 0xFFu;
    const u32x2 q = r.q[j >> 1];
    const uint32_t n0 = (j & 1) ? (q.x >> 4) & 0x0F0F0F0Fu : q.x & 0x0F0F0F0Fu;
    const uint32_t n1 = (j & 1) ? (q.y >> 4) & 0x0F0F0F0Fu : q.y & 0x0F0F0F0Fu;
    float v[8];
    // nibbles 0..15 read as fp8 are exactly n * 2^-9; v = sc * n exactly
    const float sc9 = sc * 512.f;
#pragma unroll
    for (int w = 0; w < 2; w++) {
        const uint32_t nn = w ? n1 : n0;
        const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)nn, false);
        const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)nn, true);
        v[4 * w + 0] = p0[0] * sc9;
        v[4 * w + 1] = p0[1] * sc9;
        v[4 * w + 2] = p1[0] * sc9;
        v[4 * w + 3] = p1[1] * sc9;
    }
    PfB b;
    split8(v, b.h, b.l);
    // minimum term: B = mn over the whole sub-block (bf16 of a 6-bit integer)
    const uint32_t mb = __builtin_bit_cast(uint32_t, (float)mn) >> 16;
    b.m = u32x4{mb | (mb << 16), mb | (mb << 16), mb | (mb << 16), mb | (mb << 16)};
    return b;
}

// Q6_K columns 32kc ..: v = sc * (q - 32), split exactly.
__device__ __forceinline__ PfB pf_dec(const PfRaw<Q6_K> &r, const uint32_t (&sw)[4], int kc, int c) {
    const uint32_t mis = r.mis;
    const int h = kc >> 2, k = kc & 3, hp = 2 * h + (k & 1);
    // this lane's 8 weights are l = 8c .. 8c+7 of quarter k: scale group 8h + 2k + c/2
    const int gi = 8 * h + 2 * k + (c >> 1);
    const float sc = (float)(int)(int8_t)(sw[gi >> 2] >> (8 * (gi & 3)));
    const u32x4 A = r.ql[hp], H = r.qh[h];
    const uint32_t a0 = align_bytes(A.y, A.x, mis), a1 = align_bytes(A.z, A.y, mis);
    const uint32_t h0 = align_bytes(H.y, H.x, mis), h1 = align_bytes(H.z, H.y, mis);
    const int ns = k >= 2 ? 4 : 0;
    const uint32_t q0 = ((a0 >> ns) & 0x0F0F0F0Fu) | (((h0 >> (2 * k)) & 0x03030303u) << 4);
    const uint32_t q1 = ((a1 >> ns) & 0x0F0F0F0Fu) | (((h1 >> (2 * k)) & 0x03030303u) << 4);
    float v[8];
    const float off = -32.f * sc;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        v[e] = (float)((q0 >> (8 * e)) & 0xFFu) * sc + off;  // sc * (q - 32), exact
        v[4 + e] = (float)((q1 >> (8 * e)) & 0xFFu) * sc + off;
    }
    PfB b;
    split8(v, b.h, b.l);
    b.m = b.h;
    return b;
}

// Software pipeline over the 8 chunks of a super-block: while the MFMAs of
// chunk j run, the X operands of chunk j + 1 are read from LDS and its
// weights decoded. The scheduling groups interleave one MFMA with a few VALU
// instructions, so that the matrix core and the vector ALU work together.
template <bool MIN, int VPM>
__device__ __forceinline__ void pf_issue(const bf16x8 (&av)[4], const PfB &b, f32x4 (&ah)[4], f32x4 (&al)[4],
                                         f32x4 (&am)[4]) {
    pf_chunk<MIN>(av, b.h, b.l, b.m, ah, al, am);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // the 4 X reads of the next chunk first
#pragma unroll
    for (int i = 0; i < (MIN ? 12 : 8); i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);    // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);  // then VPM VALU
    }
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void pf_mma(const PfRaw<Q4_K> &r, const uint16_t *xt, int lane, f32x4 (&out)[4]) {
    const PfScalesQ4K S = pf_scales(r);
    f32x4 ah[4], al[4], am[4];
#pragma unroll
    for (int a = 0; a < 4; a++) ah[a] = al[a] = am[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 av[2][4];
    PfB b[2];
    pf_xa(xt, lane, 0, av[0]);
    b[0] = pf_dec(r, S, 0);
#pragma unroll
    for (int j = 0; j < 8; j++) {  // sub-block j: columns 32j .. 32j+31
        if (j + 1 < 8) {
            pf_xa(xt, lane, 32 * (j + 1), av[(j + 1) & 1]);
            b[(j + 1) & 1] = pf_dec(r, S, j + 1);
        }
        pf_issue<true, 3>(av[j & 1], b[j & 1], ah, al, am);
    }
    const u32x4 h = r.h;
    const float d = half_bits_to_float(h.x & 0xFFFFu), dmin = half_bits_to_float(h.x >> 16);
#pragma unroll
    for (int a = 0; a < 4; a++) {
        out[a] += d * (ah[a] + al[a]);
        out[a] -= dmin * am[a];
    }
}

__device__ __forceinline__ void pf_mma(const PfRaw<Q6_K> &r, const uint16_t *xt, int lane, f32x4 (&out)[4]) {
    const int c = lane >> 4;
    const uint32_t mis = r.mis;
    const uint32_t sw[4] = {align_bytes(r.s.y, r.s.x, mis), align_bytes(r.s.z, r.s.y, mis),
                            align_bytes(r.s.w, r.s.z, mis), align_bytes(r.s4, r.s.w, mis)};
    f32x4 ah[4], al[4];
#pragma unroll
    for (int a = 0; a < 4; a++) ah[a] = al[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 av[2][4];
    PfB b[2];
    pf_xa(xt, lane, 0, av[0]);
    b[0] = pf_dec(r, sw, 0, c);
#pragma unroll
    for (int kc = 0; kc < 8; kc++) {  // columns 32kc .. : half h, quarter k
        if (kc + 1 < 8) {
            pf_xa(xt, lane, 32 * (kc + 1), av[(kc + 1) & 1]);
            b[(kc + 1) & 1] = pf_dec(r, sw, kc + 1, c);
        }
        pf_issue<false, 6>(av[kc & 1], b[kc & 1], ah, al, al);
    }
    const float d = half_bits_to_float(r.s4 >> 16);
#pragma unroll
    for (int a = 0; a < 4; a++) out[a] += d * (ah[a] + al[a]);
}

// KSP = 2 splits the super-blocks of the row over two halves of a 512-thread
// workgroup (waves 0-3 and 4-7, each with its own X tiles), so that two waves
// share each SIMD where the grid alone would give one; the second half's sums
// are added to the first's through LDS at the end, in a fixed order.
template <int F, int KSP>
__global__ __launch_bounds__(256 * KSP, 2 / KSP) void gemm_prefill_kernel(const uint8_t *__restrict__ W, int rows,
                                                                        int nb, int64_t row_bytes,
                                                                        const uint16_t *__restrict__ X, int M,
                                                                        float *__restrict__ Y) {
    constexpr int BYTES = Layout<F>::BYTES;
    __shared__ __attribute__((aligned(16))) uint16_t xs_all[KSP][2][PF_TM * PF_LROW];
    const int half = KSP > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 8) : 0;
    const int tid = threadIdx.x & 255, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    auto &xs = xs_all[half];
    const int c = lane >> 4;
    const int m0 = (int)blockIdx.y * PF_TM;
    const int rbase = (int)blockIdx.x * 64 + wave * 16;
    const uint8_t *const wrow = W + (int64_t)min(rbase + (lane & 15), rows - 1) * row_bytes;
    const int64_t ldx = (int64_t)nb * 256;  // X row pitch in bf16
    // this half's super-blocks [kb0, kb1); both halves run nsteps steps (the
    // second half's last one is empty when nb is odd)
    const int nh = (nb + KSP - 1) / KSP;
    const int kb0 = half * nh, kb1 = min(nb, kb0 + nh);
    const int nsteps = nh;

    // X tile staging: thread tid moves 16-byte chunks tid + 256 i (i < 8):
    // token id >> 5, k chunk id & 31; tokens past M are zero. The loads are
    // unconditional (the token is clamped into X and the value cleared
    // afterwards): a load under a branch would make the compiler wait for
    // every outstanding load, including the next step's prefetch.
    u32x4 xp[8];
    auto x_load = [&](int kb) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int id = tid + 256 * i, mr = id >> 5, kc = id & 31, m = min(m0 + mr, M - 1);
            xp[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)m * ldx + (int64_t)kb * 256 + 8 * kc);
        }
    };
    auto x_store = [&](int buf) {
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int id = tid + 256 * i, mr = id >> 5, kc = id & 31;
            const uint32_t keep = m0 + mr < M ? 0xFFFFFFFFu : 0u;
            *reinterpret_cast<u32x4 *>(&xs[buf][mr * PF_LROW + 8 * kc]) = xp[i] & keep;
        }
    };

    f32x4 acc[4];
#pragma unroll
    for (int a = 0; a < 4; a++) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The next step's weights and X tile load while this step is multiplied
    // (two register buffers for the weights, two LDS buffers for X).
    PfRaw<F> wb[2];
    const int klast = kb1 - 1;  // >= kb0 for every half that has work
    x_load(min(kb0, nb - 1));
    pf_load(wb[0], wrow + (int64_t)min(kb0, nb - 1) * BYTES, c);
    x_store(0);
    __syncthreads();
    // The prefetch is unconditional (past this half's last step it reloads
    // that block): loads under a branch would make the compiler wait for all
    // of them.
    auto step = [&](int i, PfRaw<F> &cur, PfRaw<F> &next, int xb) {
        const int kb = kb0 + i;
        const int kn = max(min(kb + 1, klast), 0);
        x_load(kn);
        pf_load(next, wrow + (int64_t)kn * BYTES, c);
        __builtin_amdgcn_sched_barrier(0);
        if (kb < kb1) pf_mma(cur, xs[xb], lane, acc);
        if (i + 1 < nsteps) x_store(xb ^ 1);
        __syncthreads();
    };
    for (int i = 0; i < nsteps; i += 2) {
        step(i, wb[0], wb[1], 0);
        if (i + 1 >= nsteps) break;
        step(i + 1, wb[1], wb[0], 1);
    }

    // lane holds tokens 16a + 4c + i of row rbase + lane % 16
    if constexpr (KSP > 1) {
        // the second half's sums go through LDS (over its X tiles) to the first
        float *part = reinterpret_cast<float *>(&xs_all[1][0][0]);
        if (half == 1) {
#pragma unroll
            for (int a = 0; a < 4; a++) *reinterpret_cast<f32x4 *>(part + (tid * 4 + a) * 4) = acc[a];
        }
        __syncthreads();
        if (half == 1) return;
#pragma unroll
        for (int a = 0; a < 4; a++) acc[a] += *reinterpret_cast<const f32x4 *>(part + (tid * 4 + a) * 4);
    }
    const int r = rbase + (lane & 15);
#pragma unroll
    for (int a = 0; a < 4; a++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = m0 + 16 * a + 4 * c + i;
            if (m < M && r < rows) Y[(int64_t)m * rows + r] = acc[a][i];
        }
}

template <int F, int KSP>
static hipError_t launch_prefill(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                                 int64_t M, float *Y, hipStream_t stream) {
    const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((M + PF_TM - 1) / PF_TM));
    hipLaunchKernelGGL((gemm_prefill_kernel<F, KSP>), grid, dim3(256 * KSP), 0, stream, W, (int)rows,
                       (int)(cols / 256), row_bytes, X, (int)M, Y);
    return hipGetLastError();
}

// Which kernel a GEMM of this format, shape and M runs (a qk_gemm_path):
// the row kernel for every format but Q4_K and Q6_K, else the few-token
// kernel for M <= 16 and the prefill kernel above. QK_TUNE_GEMM_PATH forces
// one where it applies (the few-token kernel takes at most 16 rows of X).
template <int F> static int gemm_path_t(int64_t rows, int64_t cols, int64_t M) {
    (void)cols;
    if constexpr (F == Q4_K || F == Q6_K) {
        if (rows < (int64_t(1) << 30) && M < (int64_t(1) << 30)) {
            const int force = tuning(QK_TUNE_GEMM_PATH);
            if (force == QK_GEMM_PATH_ROWS) return QK_GEMM_PATH_ROWS;
            if (force == QK_GEMM_PATH_PREFILL) return QK_GEMM_PATH_PREFILL;
            if (force == QK_GEMM_PATH_FEW && M <= 16) return QK_GEMM_PATH_FEW;
            return M <= 16 ? QK_GEMM_PATH_FEW : QK_GEMM_PATH_PREFILL;
        }
    }
    return QK_GEMM_PATH_ROWS;
}

template <int F>
static hipError_t launch_gemm_t(const uint8_t *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M, float *Y,
                                hipStream_t stream) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    const int64_t row_bytes = cols / QK * BYTES;
    const int path = gemm_path_t<F>(rows, cols, M);
    if constexpr (F == Q4_K || F == Q6_K) {
        if (path == QK_GEMM_PATH_PREFILL) {
            // Two halves of the super-blocks per workgroup when the grid alone
            // gives at most one workgroup per CU (then two waves share each
            // SIMD): measured at M = 64..512 on the 5632 x 2048 and 2048 x 5632
            // shapes. QK_TUNE_GEMM_KSPLIT = 1/2 forces it.
            const int64_t wgs = ((rows + 63) / 64) * ((M + PF_TM - 1) / PF_TM);
            const int ksf = tuning(QK_TUNE_GEMM_KSPLIT);
            const bool split = cols / QK >= 2 && (ksf == 2 || (ksf < 0 && wgs <= device_cu_count()));
            return split ? launch_prefill<F, 2>(W, rows, cols, row_bytes, X, M, Y, stream)
                         : launch_prefill<F, 1>(W, rows, cols, row_bytes, X, M, Y, stream);
        }
        if (path == QK_GEMM_PATH_FEW) return launch_few<F>(W, rows, cols, row_bytes, X, M, Y, stream);
    }
    constexpr int MB = 8;
    const int64_t jobs = rows * ((M + MB - 1) / MB);
    int64_t grid = (jobs + 3) / 4;
    const int64_t cap = (int64_t)device_cu_count() * 16;
    if (grid > cap) grid = cap;
    hipLaunchKernelGGL((gemm_rows_kernel<F, MB>), dim3((unsigned)grid), dim3(256), 0, stream, W, rows, cols, row_bytes,
                       X, M, Y);
    return hipGetLastError();
}

int gemm_path(int type, int64_t rows, int64_t cols, int64_t M) {
    switch (type) {
    case Q4_K: return gemm_path_t<Q4_K>(rows, cols, M);
    case Q6_K: return gemm_path_t<Q6_K>(rows, cols, M);
    default: return 0;
    }
}

hipError_t launch_gemm(int type, const void *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M, float *Y,
                       hipStream_t stream) {
    const uint8_t *w = static_cast<const uint8_t *>(W);
    switch (type) {
    case Q4_K: return launch_gemm_t<Q4_K>(w, rows, cols, X, M, Y, stream);
    case Q6_K: return launch_gemm_t<Q6_K>(w, rows, cols, X, M, Y, stream);
    case Q8_0: return launch_gemm_t<Q8_0>(w, rows, cols, X, M, Y, stream);
    case Q4_0: return launch_gemm_t<Q4_0>(w, rows, cols, X, M, Y, stream);
    case Q8_0_F16: return launch_gemm_t<Q8_0_F16>(w, rows, cols, X, M, Y, stream);
    case Q5_1: return launch_gemm_t<Q5_1>(w, rows, cols, X, M, Y, stream);
    case Q5_K: return launch_gemm_t<Q5_K>(w, rows, cols, X, M, Y, stream);
    case Q2_K: return launch_gemm_t<Q2_K>(w, rows, cols, X, M, Y, stream);
    case Q3_K: return launch_gemm_t<Q3_K>(w, rows, cols, X, M, Y, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qk
