// qk_gemm.hip — Y = X W^T for M activation rows (bf16 X, fp32 Y).
//
// Batched path: one wave per weight row; lanes walk the row four weights at a
// time with the bit-exact decoder and accumulate up to MB activation rows at
// once, so W is streamed once per MB rows of X.
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

// ---------------------------------------------------------------------------
// MFMA tile kernel (multi-token prefill).
//
// Y[m, r] = sum_k X[m, k] w[r, k] is a dense contraction, so it runs on the
// matrix cores. The weights enter the MFMA as their exact integer codes in
// bf16 (Q4_K q in 0..15, Q6_K q in -32..31 are exact in bf16's 8-bit
// significand); X enters as given (bf16). Each MFMA spans one scale group —
// 32 columns of a Q4_K sub-block (v_mfma_f32_16x16x32_bf16) or 16 columns of
// a Q6_K group (v_mfma_f32_16x16x16_bf16) — and its fp32 result is scaled by
// that group's d*scale (and, for Q4_K, the group's dmin*min times the sum of
// X over the group is subtracted) in fp32. So no weight is ever rounded to
// bf16: rounding dequantised weights to bf16 would exceed the tolerance.
//
// Workgroup tile: TM = 16*MTW*WM rows of X by TR = 16*RTW*WR weight rows,
// 64*WM*WR threads; one K step is one super-block (256 columns): the X tile
// and the decoded code tile are staged in LDS (rows padded by 16 bytes so
// the 16-byte fragment reads are bank-conflict free), then every wave runs
// its MTW x RTW MFMA tiles over the block's scale groups.
// ---------------------------------------------------------------------------

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int F> struct Groups;
template <> struct Groups<Q4_K> { static constexpr int N = 8, K = 32; };   // sub-blocks of 32
template <> struct Groups<Q6_K> { static constexpr int N = 16, K = 16; };  // scale groups of 16

constexpr int KSTEP = 256;            // one super-block per K step
constexpr int LROW = KSTEP + 8;       // LDS row pitch in bf16 (16 bytes of padding)

__device__ __forceinline__ uint32_t bf16_of_small_int(uint32_t v) {
    // integer |v| < 2^8 -> its bf16 bit pattern (exact): the top half of the fp32
    return __builtin_bit_cast(uint32_t, (float)(int)v) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (__builtin_bit_cast(uint32_t, lo) >> 16) | (__builtin_bit_cast(uint32_t, hi) & 0xFFFF0000u);
}

// Decode one 64-weight unit of row `r` of the block at `blk` into LDS codes
// (bf16) and per-group scales. Q4_K unit u = nibble group g (sub-blocks 2g,
// 2g+1); Q6_K unit u = (half h, 16 positions l0) x 4 quarters.
template <int F>
__device__ __forceinline__ void decode_unit_to_lds(const uint8_t *blk, int u, uint16_t *wrow, float *srow, float *mrow);

template <>
__device__ __forceinline__ void decode_unit_to_lds<Q4_K>(const uint8_t *blk, int g, uint16_t *wrow, float *srow,
                                                          float *mrow) {
    const u32x4 h = ld_b128(blk);
    const u32x4 qa = ld_b128(blk + 16 + 32 * g), qb = ld_b128(blk + 32 + 32 * g);
    const uint32_t q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
    // codes: low nibbles -> k = 64g + l, high nibbles -> k = 64g + 32 + l
#pragma unroll
    for (int half = 0; half < 2; half++) {
        uint32_t packed[16];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const uint32_t w = (q[i] >> (4 * half)) & 0x0F0F0F0Fu;
            const float f0 = (float)(w & 0xFFu), f1 = (float)((w >> 8) & 0xFFu);
            const float f2 = (float)((w >> 16) & 0xFFu), f3 = (float)(w >> 24);
            packed[2 * i] = pack_bf16(f0, f1);
            packed[2 * i + 1] = pack_bf16(f2, f3);
        }
        uint32_t *dst = reinterpret_cast<uint32_t *>(wrow + 64 * g + 32 * half);
#pragma unroll
        for (int i = 0; i < 16; i += 4)
            *reinterpret_cast<u32x4 *>(dst + i) = u32x4{packed[i], packed[i + 1], packed[i + 2], packed[i + 3]};
    }
    uint32_t s0, m0, s1, m1;
    q4k_scale_min(h.y, h.z, h.w, 2 * g, s0, m0);
    q4k_scale_min(h.y, h.z, h.w, 2 * g + 1, s1, m1);
    const float d = half_bits_to_float(h.x & 0xFFFFu), dmin = half_bits_to_float(h.x >> 16);
    srow[2 * g] = d * (float)s0;
    srow[2 * g + 1] = d * (float)s1;
    mrow[2 * g] = dmin * (float)m0;
    mrow[2 * g + 1] = dmin * (float)m1;
}

template <>
__device__ __forceinline__ void decode_unit_to_lds<Q6_K>(const uint8_t *blk, int u, uint16_t *wrow, float *srow,
                                                          float *) {
    const int h = u >> 1, l0 = 16 * (u & 1);
    // 2-byte loads: Q6_K blocks are only 2-byte aligned in general
    uint32_t A[4], B[4], H[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        A[i] = ld_u32_via_u16(blk + 64 * h + l0 + 4 * i);
        B[i] = ld_u32_via_u16(blk + 64 * h + 32 + l0 + 4 * i);
        H[i] = ld_u32_via_u16(blk + 128 + 32 * h + l0 + 4 * i);
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t packed[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t lo = ((k & 1 ? B[i] : A[i]) >> (k >= 2 ? 4 : 0)) & 0x0F0F0F0Fu;
            const uint32_t c = lo | (((H[i] >> (2 * k)) & 0x03030303u) << 4);  // 6-bit codes
            const float f0 = (float)((int)(c & 0xFFu) - 32), f1 = (float)((int)((c >> 8) & 0xFFu) - 32);
            const float f2 = (float)((int)((c >> 16) & 0xFFu) - 32), f3 = (float)((int)(c >> 24) - 32);
            packed[2 * i] = pack_bf16(f0, f1);
            packed[2 * i + 1] = pack_bf16(f2, f3);
        }
        uint32_t *dst = reinterpret_cast<uint32_t *>(wrow + 128 * h + 32 * k + l0);
        *reinterpret_cast<u32x4 *>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
        *reinterpret_cast<u32x4 *>(dst + 4) = u32x4{packed[4], packed[5], packed[6], packed[7]};
    }
    const float d = half_bits_to_float(ld_b16(blk + 208));
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int gi = 8 * h + 2 * k + (l0 >> 4);  // one scale per 16 weights
        const uint32_t pr = ld_b16(blk + 192 + (gi & ~1));
        srow[gi] = d * (float)(int)(int8_t)(pr >> (8 * (gi & 1)));
    }
}

template <int F, int MTW, int RTW, int WM, int WR>
__global__ __launch_bounds__(64 * WM * WR) void gemm_mfma_kernel(const uint8_t *__restrict__ W, int64_t rows,
                                                                int64_t cols, int64_t row_bytes,
                                                                const uint16_t *__restrict__ X, int64_t M,
                                                                float *__restrict__ Y) {
    constexpr int NT = 64 * WM * WR;
    constexpr int TM = 16 * MTW * WM, TR = 16 * RTW * WR;
    constexpr int NG = Groups<F>::N, GK = Groups<F>::K;
    constexpr int BYTES = Layout<F>::BYTES;
    __shared__ __attribute__((aligned(16))) uint16_t xs[TM * LROW];
    __shared__ __attribute__((aligned(16))) uint16_t ws[TR * LROW];
    __shared__ float ssc[TR * NG];  // d * scale per (row, group)
    __shared__ float smn[F == Q4_K ? TR * NG : 1];  // dmin * min per (row, group)
    __shared__ __attribute__((aligned(16))) float xsum[F == Q4_K ? NG * TM : 4];  // sum of X per (group, m)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / WR, wr = wave % WR;
    const int64_t m0 = (int64_t)blockIdx.y * TM, r0 = (int64_t)blockIdx.x * TR;

    f32x4 acc[MTW][RTW];
#pragma unroll
    for (int a = 0; a < MTW; a++)
#pragma unroll
        for (int b = 0; b < RTW; b++) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t nblk = cols / KSTEP;
    for (int64_t kb = 0; kb < nblk; kb++) {
        __syncthreads();  // the previous step's LDS reads are done
        // X tile: TM rows x 256 bf16, 16-byte chunks, consecutive threads on
        // consecutive chunks; rows past M are zero.
        for (int c = tid; c < TM * 32; c += NT) {
            const int mr = c >> 5, kc = c & 31;
            const int64_t m = m0 + mr;
            u32x4 v = u32x4{0u, 0u, 0u, 0u};
            if (m < M) v = *reinterpret_cast<const u32x4 *>(X + m * cols + kb * KSTEP + 8 * kc);
            *reinterpret_cast<u32x4 *>(xs + mr * LROW + 8 * kc) = v;
            if (F == Q4_K) {
                // sum of the 8 values, then over the 4 chunks of a sub-block (lanes 4s..4s+3)
                float t = bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) + bf16_lo(v.z) + bf16_hi(v.z) +
                          bf16_lo(v.w) + bf16_hi(v.w);
                t += __shfl_xor(t, 1);
                t += __shfl_xor(t, 2);
                if ((kc & 3) == 0) xsum[(kc >> 2) * TM + mr] = t;
            }
        }
        // Decoded codes and scales of TR weight rows (4 units of 64 weights per row).
        for (int c = tid; c < TR * 4; c += NT) {
            const int rr = c >> 2, u = c & 3;
            const int64_t r = min(r0 + rr, rows - 1);
            decode_unit_to_lds<F>(W + r * row_bytes + kb * BYTES, u, ws + rr * LROW, ssc + rr * NG, smn + rr * NG);
        }
        __syncthreads();

#pragma unroll
        for (int gi = 0; gi < NG; gi++) {
#pragma unroll
            for (int a = 0; a < MTW; a++) {
                const int mrow = 16 * (wm * MTW + a) + (lane & 15);
#pragma unroll
                for (int b = 0; b < RTW; b++) {
                    const int rrow = 16 * (wr * RTW + b) + (lane & 15);
                    f32x4 p;
                    if (GK == 32) {
                        const int kofs = 32 * gi + 8 * (lane >> 4);
                        const bf16x8 av = *reinterpret_cast<const bf16x8 *>(xs + mrow * LROW + kofs);
                        const bf16x8 bv = *reinterpret_cast<const bf16x8 *>(ws + rrow * LROW + kofs);
                        p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    } else {
                        const int kofs = 16 * gi + 4 * (lane >> 4);
                        const s16x4 av = *reinterpret_cast<const s16x4 *>(xs + mrow * LROW + kofs);
                        const s16x4 bv = *reinterpret_cast<const s16x4 *>(ws + rrow * LROW + kofs);
                        p = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
                    }
                    // this lane's outputs: rows m = 16*(wm*MTW+a) + 4*(lane/16) + i, column rrow
                    const float sc = ssc[rrow * NG + gi];
                    acc[a][b] += sc * p;
                    if (F == Q4_K) {
                        const float mn = smn[rrow * NG + gi];
                        const f32x4 xv =
                            *reinterpret_cast<const f32x4 *>(xsum + gi * TM + 16 * (wm * MTW + a) + 4 * (lane >> 4));
                        acc[a][b] -= mn * xv;
                    }
                }
            }
        }
    }

    // Y[m][r]: this lane holds rows 4*(lane/16)+i of each 16x16 tile, column lane%16.
#pragma unroll
    for (int a = 0; a < MTW; a++)
#pragma unroll
        for (int b = 0; b < RTW; b++) {
            const int64_t r = r0 + 16 * (wr * RTW + b) + (lane & 15);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int64_t m = m0 + 16 * (wm * MTW + a) + 4 * (lane >> 4) + i;
                if (m < M && r < rows) Y[m * rows + r] = acc[a][b][i];
            }
        }
}

template <int F, int MTW, int RTW, int WM, int WR>
static hipError_t launch_mfma(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                              int64_t M, float *Y, hipStream_t stream) {
    constexpr int TM = 16 * MTW * WM, TR = 16 * RTW * WR;
    const dim3 grid((unsigned)((rows + TR - 1) / TR), (unsigned)((M + TM - 1) / TM));
    hipLaunchKernelGGL((gemm_mfma_kernel<F, MTW, RTW, WM, WR>), grid, dim3(64 * WM * WR), 0, stream, W, rows, cols,
                       row_bytes, X, M, Y);
    return hipGetLastError();
}

template <int F>
static hipError_t launch_gemm_t(const uint8_t *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M, float *Y,
                                hipStream_t stream) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    const int64_t row_bytes = cols / QK * BYTES;
    if constexpr (F == Q4_K || F == Q6_K) {
        const char *e = getenv("QK_GEMM_PATH");  // sweep override: 0 rows, 1 large tile, 2 small tile
        const int path = (e && *e) ? atoi(e) : -1;
        if (path == 1 || (path < 0 && M > 16)) {
            return launch_mfma<F, 2, 2, 2, 2>(W, rows, cols, row_bytes, X, M, Y, stream);
        }
        if (path == 2) return launch_mfma<F, 1, 1, 1, 4>(W, rows, cols, row_bytes, X, M, Y, stream);
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

hipError_t launch_gemm(int type, const void *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M, float *Y,
                       hipStream_t stream) {
    const uint8_t *w = static_cast<const uint8_t *>(W);
    switch (type) {
    case Q4_K: return launch_gemm_t<Q4_K>(w, rows, cols, X, M, Y, stream);
    case Q6_K: return launch_gemm_t<Q6_K>(w, rows, cols, X, M, Y, stream);
    case Q8_0: return launch_gemm_t<Q8_0>(w, rows, cols, X, M, Y, stream);
    case Q4_0: return launch_gemm_t<Q4_0>(w, rows, cols, X, M, Y, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace qk
