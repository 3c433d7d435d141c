// qk_gemm.hip — Y = X W^T for M activation rows (bf16 X, fp32 Y).
//
// The multi-token path ("picoLM, in Python" prefills one position at a time;
// batching positions turns the GEMV into a dense contraction):
// * gemm_few_kernel (1 < M <= 16, K-quants): W streams once through the
//   MFMA, codes exact in bf16, scales applied per group in fp32;
// * gemm_pw_kernel (M > 16, Q4_K and Q6_K): 64 rows x 64 tokens per
//   workgroup, X tiles double-buffered in LDS; each wave decodes its weight
//   rows into bf16 hi/lo operands (two MFMAs per product);
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

// ---------------------------------------------------------------------------
// Prefill kernel (M > 16, Q4_K and Q6_K).
//
// A workgroup computes 64 weight rows x 64 tokens; each of its 4 waves owns
// 16 rows and all 64 tokens (4 M tiles of v_mfma_f32_16x16x32_bf16). K
// advances 128 columns (half a super-block) per step; the step's 64 x 128
// bf16 X tile sits in LDS (double-buffered, 34 KiB), and lane (n, c) reads
// the A operand of token 16a + n at columns 8c..8c+7 of each 32-column
// chunk, the B operand of its row n at the same columns. (128 tokens per
// workgroup, each decoded weight feeding 8 tiles, measured no faster at
// M = 512 on the 5632 x 2048, 2048 x 5632 and 4096 x 11008 shapes, and
// slower at M = 64.)
//
// Operands (two MFMAs per product, X * hi + X * lo, fp32 accumulation):
//   Q6_K  v = sc * (q - 32), an integer of at most 13 bits, split exactly
//         into bf16 v_hi + v_lo; every product is exact and the super-block's
//         d multiplies the sums of its two steps;
//   Q4_K  w = (d*sc)*q - dmin*mn in fp32 (one rounding), split into
//         w_hi = w rounded to bf16 and w_lo = (w - w_hi) rounded to bf16:
//         |w - w_hi - w_lo| <= 2^-16 |w|, so the result stays within
//         2^-16 * sum|w*x| of the exact products' sum (plus the fp32
//         accumulation), far inside the tolerance for any input; the
//         minimum term needs no third MFMA.
//
// KH = 2 splits K over two workgroups (blockIdx.z) that add their sums
// into Y, which a fill launch zeroes first (two addends to zero: the order
// does not change the result); used where the row and token tiles alone
// leave CUs idle (the 2048 x 5632 down shape).
// ---------------------------------------------------------------------------

constexpr int PW_TOK = 64;   // tokens per workgroup
constexpr int PW_LX = 136;   // LDS row pitch of the X tile (bf16): 128 + 8

// fp32 -> bf16 with ties rounded up in magnitude: adding half a bf16 ulp to
// the pattern, then keeping the top 16 bits
__device__ __forceinline__ uint32_t bf16_round_bits(float v) { return __builtin_bit_cast(uint32_t, v) + 0x8000u; }

// Raw bytes of one half super-block for lane (n, c).
template <int F> struct PwRaw;
template <> struct PwRaw<Q4_K> {
    u32x4 h;     // d | dmin | packed scales and mins
    u32x2 q[2];  // nibble bytes 32g + 8c .. +7 of the half's two nibble groups
};
template <> struct PwRaw<Q6_K> {
    u32x4 ql[2];  // ql windows 64h + 32p + 8c (p = 0, 1), from the 4-byte boundary below
    u32x4 qh;     // qh window 128 + 32h + 8c
    u32x4 s;      // scales window
    uint32_t s4;  // q6k_tail: scales 14, 15 and d
    uint32_t mis; // bytes from the 4-byte boundary below the block to it (0 or 2)
};

__device__ __forceinline__ void pw_load(PwRaw<Q4_K> &r, const uint8_t *blk, int h, int c) {
    r.h = ld_b128(blk);
#pragma unroll
    for (int i = 0; i < 2; i++) r.q[i] = ld_b64(blk + 16 + 32 * (2 * h + i) + 8 * c);
}

__device__ __forceinline__ void pw_load(PwRaw<Q6_K> &r, const uint8_t *blk, int h, int c) {
    r.mis = (uint32_t)(uintptr_t)blk & 3u;
    const uint8_t *A0 = blk - r.mis;
#pragma unroll
    for (int p = 0; p < 2; p++) r.ql[p] = ld_b128(A0 + 64 * h + 32 * p + 8 * c);
    r.qh = ld_b128(A0 + 128 + 32 * h + 8 * c);
    r.s = ld_b128(A0 + 192);
    r.s4 = q6k_tail(blk);
}

// B operands (hi, lo) of chunk j (columns 32j.. of the half) for lane c.
__device__ __forceinline__ void pw_dec(const PwRaw<Q4_K> &r, int h, int j, u32x4 &bh, u32x4 &bl) {
    const u32x4 hd = r.h;
    // sub-block s = 4h + j: nibble group 2h + j/2, low nibbles for even s
    const int sb = 4 * h + j;
    const uint32_t sc_lo = hd.y & 0x3F3F3F3Fu, mn_lo = hd.z & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t mn_hi = ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
    const uint32_t SC = sb < 4 ? sc_lo : sc_hi, MN = sb < 4 ? mn_lo : mn_hi;
    const float d = half_bits_to_float(hd.x & 0xFFFFu), dmin = half_bits_to_float(hd.x >> 16);
    // nibbles read as fp8 are n * 2^-9: a = d * sc * 512 (exact), b = dmin * mn
    const float a = d * (float)((SC >> (8 * (sb & 3))) & 0xFFu) * 512.f;
    const float b = dmin * (float)((MN >> (8 * (sb & 3))) & 0xFFu);
    const u32x2 q = r.q[j >> 1];
    const uint32_t n0 = (j & 1) ? (q.x >> 4) & 0x0F0F0F0Fu : q.x & 0x0F0F0F0Fu;
    const uint32_t n1 = (j & 1) ? (q.y >> 4) & 0x0F0F0F0Fu : q.y & 0x0F0F0F0Fu;
    float w[8];
#pragma unroll
    for (int k = 0; k < 2; k++) {
        const uint32_t nn = k ? n1 : n0;
        const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)nn, false);
        const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)nn, true);
        w[4 * k + 0] = __builtin_fmaf(a, p0[0], -b);
        w[4 * k + 1] = __builtin_fmaf(a, p0[1], -b);
        w[4 * k + 2] = __builtin_fmaf(a, p1[0], -b);
        w[4 * k + 3] = __builtin_fmaf(a, p1[1], -b);
    }
    uint32_t hb[8], lb[8];
#pragma unroll
    for (int e = 0; e < 8; e++) {
        hb[e] = bf16_round_bits(w[e]);
        const float hi = __builtin_bit_cast(float, hb[e] & 0xFFFF0000u);
        lb[e] = bf16_round_bits(w[e] - hi);
    }
    // top halves of two patterns as one bf16 pair
    auto top2 = [](uint32_t lo, uint32_t hi) { return __builtin_amdgcn_perm(hi, lo, 0x07060302u); };
    bh = u32x4{top2(hb[0], hb[1]), top2(hb[2], hb[3]), top2(hb[4], hb[5]), top2(hb[6], hb[7])};
    bl = u32x4{top2(lb[0], lb[1]), top2(lb[2], lb[3]), top2(lb[4], lb[5]), top2(lb[6], lb[7])};
}

__device__ __forceinline__ void pw_dec(const PwRaw<Q6_K> &r, int h, int j, int c, u32x4 &bh, u32x4 &bl) {
    const uint32_t mis = r.mis;
    // quarter j of half h: ql window p = j & 1 (low nibbles for j < 2), qh bits 2j
    const u32x4 A = r.ql[j & 1], H = r.qh;
    const uint32_t a0 = align_bytes(A.y, A.x, mis), a1 = align_bytes(A.z, A.y, mis);
    const uint32_t h0 = align_bytes(H.y, H.x, mis), h1 = align_bytes(H.z, H.y, mis);
    const int ns = j >= 2 ? 4 : 0;
    const uint32_t q0 = ((a0 >> ns) & 0x0F0F0F0Fu) | (((h0 >> (2 * j)) & 0x03030303u) << 4);
    const uint32_t q1 = ((a1 >> ns) & 0x0F0F0F0Fu) | (((h1 >> (2 * j)) & 0x03030303u) << 4);
    // this lane's 8 weights l = 8c..8c+7 of the quarter: scale 8h + 2j + c/2
    const int gi = 8 * h + 2 * j + (c >> 1);
    const uint32_t sw = gi < 12 ? align_bytes(gi < 4 ? r.s.y : gi < 8 ? r.s.z : r.s.w,
                                              gi < 4 ? r.s.x : gi < 8 ? r.s.y : r.s.z, mis)
                                : align_bytes(r.s4, r.s.w, mis);
    const float sc = (float)(int)(int8_t)(sw >> (8 * (gi & 3)));
    const float off = -32.f * sc;
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        v[e] = __builtin_fmaf((float)((q0 >> (8 * e)) & 0xFFu), sc, off);  // sc * (q - 32), exact
        v[4 + e] = __builtin_fmaf((float)((q1 >> (8 * e)) & 0xFFu), sc, off);
    }
    split8(v, bh, bl);
}

template <int F, int KH>
__global__ __launch_bounds__(256, F == Q6_K ? 2 : 3) void gemm_pw_kernel(const uint8_t *__restrict__ W, int rows, int nb,
                                                         int64_t row_bytes, const uint16_t *__restrict__ X, int M,
                                                         float *__restrict__ Y) {
    constexpr int BYTES = Layout<F>::BYTES;
    constexpr int PW_MT = PW_TOK / 16;  // M tiles per wave
    constexpr int XCH = PW_TOK / 16;    // 16-byte X chunks per thread and step
    __shared__ __attribute__((aligned(16))) uint16_t xs[2][PW_TOK * PW_LX];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, c = lane >> 4;
    const int m0 = (int)blockIdx.y * PW_TOK;
    const int rbase = (int)blockIdx.x * 64 + wave * 16;
    const uint8_t *const wrow = W + (int64_t)min(rbase + n, rows - 1) * row_bytes;
    const int64_t ldx = (int64_t)nb * 256;
    // this workgroup's half super-blocks [t0, t0 + nsteps): all of them, or
    // those of one of two halves of the row's super-blocks (whole super-blocks,
    // so that each one's scale applies to both its halves; the host keeps
    // nb >= 2 for KH = 2)
    const int kb0 = KH > 1 ? (int)blockIdx.z * (nb / 2) : 0;
    const int kb1 = KH > 1 && blockIdx.z == 0 ? nb / 2 : nb;
    const int nsteps = 2 * (kb1 - kb0);
    const int t0 = 2 * kb0;

    // X tile staging: thread tid moves 16-byte chunks tid + 256 i (i < XCH):
    // token id >> 4, columns 8 (id & 15) ..; tokens past M load token M - 1
    // (unconditional loads) and are cleared before the store
    u32x4 xp[2][XCH];
    auto x_load = [&](u32x4 *dst, int t) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int id = tid + 256 * i, mr = id >> 4, kc = id & 15, m = min(m0 + mr, M - 1);
            dst[i] = *reinterpret_cast<const u32x4 *>(X + (int64_t)m * ldx + (int64_t)t * 128 + 8 * kc);
        }
    };
    auto x_store = [&](const u32x4 *src, int buf) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int id = tid + 256 * i, mr = id >> 4, kc = id & 15;
            const uint32_t keep = m0 + mr < M ? 0xFFFFFFFFu : 0u;
            *reinterpret_cast<u32x4 *>(&xs[buf][mr * PW_LX + 8 * kc]) = src[i] & keep;
        }
    };
    auto w_load = [&](PwRaw<F> &r, int t) { pw_load(r, wrow + (int64_t)(t >> 1) * BYTES, t & 1, c); };

    f32x4 acc[PW_MT], sbacc[F == Q6_K ? PW_MT : 1];
#pragma unroll
    for (int a = 0; a < PW_MT; a++) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    // X and the weights are loaded two steps ahead (X tiles and L2/Infinity
    // Cache latency ~1-2 us against ~0.5 us of work per step): the X tile of
    // step t + 1 waits in registers while step t computes from LDS, and the
    // weights of steps t + 1 and t + 2 are in flight
    PwRaw<F> wb[3];
    const int tl = t0 + nsteps - 1;
    x_load(xp[0], t0);
    x_load(xp[1], min(t0 + 1, tl));
    w_load(wb[0], t0);
    w_load(wb[1], min(t0 + 1, tl));
    x_store(xp[0], 0);
    __syncthreads();

    // one step: the 4 chunks of half t, the X tile in xs[buf]
    auto compute = [&](const PwRaw<F> &r, int t, int buf) {
        const uint16_t *xt = xs[buf] + n * PW_LX + 8 * c;
        const int h = t & 1;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            u32x4 bh, bl;
            if constexpr (F == Q4_K)
                pw_dec(r, h, j, bh, bl);
            else
                pw_dec(r, h, j, c, bh, bl);
            bf16x8 av[PW_MT];
#pragma unroll
            for (int a = 0; a < PW_MT; a++) av[a] = *reinterpret_cast<const bf16x8 *>(xt + 16 * a * PW_LX + 32 * j);
            if constexpr (F == Q4_K) {
#pragma unroll
                for (int a = 0; a < PW_MT; a++)
                    acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bh), acc[a], 0, 0, 0);
#pragma unroll
                for (int a = 0; a < PW_MT; a++)
                    acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bl), acc[a], 0, 0, 0);
            } else {
                // the super-block's sums start at its first chunk
                const bool first = h == 0 && j == 0;
#pragma unroll
                for (int a = 0; a < PW_MT; a++)
                    sbacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        av[a], __builtin_bit_cast(bf16x8, bh), first ? f32x4{0.f, 0.f, 0.f, 0.f} : sbacc[a], 0, 0, 0);
#pragma unroll
                for (int a = 0; a < PW_MT; a++)
                    sbacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bl), sbacc[a],
                                                                      0, 0, 0);
            }
        }
        if constexpr (F == Q6_K) {
            if (h == 1) {  // the super-block is complete: its d scales its sums
                const float d = half_bits_to_float(r.s4 >> 16);
#pragma unroll
                for (int a = 0; a < PW_MT; a++) acc[a] += d * sbacc[a];
            }
        }
    };
    // step k of a round of 6 (the buffer indices are compile-time): loads for
    // step t + 2, the multiply of step t, then the X tile of step t + 1 into
    // the other LDS buffer; the loads are unconditional (past the last step
    // they reload it)
#define QK_PW_STEP(K)                                                           \
    {                                                                           \
        const int t = t0 + i + (K), t2 = min(t + 2, tl);                        \
        x_load(xp[(K) % 2], t2);                                                \
        w_load(wb[((K) + 2) % 3], t2);                                          \
        __builtin_amdgcn_sched_barrier(0);                                      \
        compute(wb[(K) % 3], t, (K) % 2);                                       \
        if (i + (K) + 1 < nsteps) x_store(xp[((K) + 1) % 2], ((K) + 1) % 2);  \
        __syncthreads();                                                        \
        if (i + (K) + 1 >= nsteps) break;                                       \
    }
    for (int i = 0; i < nsteps; i += 6) {
        QK_PW_STEP(0)
        QK_PW_STEP(1)
        QK_PW_STEP(2)
        QK_PW_STEP(3)
        QK_PW_STEP(4)
        QK_PW_STEP(5)
    }
#undef QK_PW_STEP

    // lane holds tokens 16a + 4c + i of row rbase + n
    const int r = rbase + n;
#pragma unroll
    for (int a = 0; a < PW_MT; a++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int m = m0 + 16 * a + 4 * c + i;
            if (m < M && r < rows) {
                if constexpr (KH == 1)
                    Y[(int64_t)m * rows + r] = acc[a][i];
                else
                    atomicAdd(&Y[(int64_t)m * rows + r], acc[a][i]);
            }
        }
}

template <int F, int KH>
static hipError_t launch_pw(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                            int64_t M, float *Y, hipStream_t stream) {
    if (KH > 1) {
        const hipError_t ez = launch_fill_zero(Y, M * rows, stream);
        if (ez != hipSuccess) return ez;
    }
    const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((M + PW_TOK - 1) / PW_TOK), (unsigned)KH);
    hipLaunchKernelGGL((gemm_pw_kernel<F, KH>), grid, dim3(256), 0, stream, W, (int)rows, (int)(cols / 256), row_bytes,
                       X, (int)M, Y);
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
            // K split over two workgroups when the row x token tiles number
            // no more than the CUs (measured at M = 64 and 512 on the 5632 x
            // 2048, 2048 x 5632 and 4096 x 11008 shapes);
            // QK_TUNE_GEMM_KSPLIT = 1/2 forces it
            const int ksf = tuning(QK_TUNE_GEMM_KSPLIT);
            const int64_t tiles = ((rows + 63) / 64) * ((M + PW_TOK - 1) / PW_TOK);
            const bool split = cols / QK >= 2 && (ksf == 2 || (ksf < 0 && tiles <= device_cu_count()));
            return split ? launch_pw<F, 2>(W, rows, cols, row_bytes, X, M, Y, stream)
                         : launch_pw<F, 1>(W, rows, cols, row_bytes, X, M, Y, stream);
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
