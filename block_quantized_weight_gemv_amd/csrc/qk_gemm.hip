// qk_gemm.hip — Y = X W^T for M activation rows (bf16 X, fp32 Y).
//
// The multi-token path ("picoLM, in Python" prefills one position at a time;
// batching positions turns the GEMV into a dense contraction):
// * gemm_few_kernel (M <= 16; rows of whole 256-column steps, every format):
//   W streams once through the MFMA; Q4_K, Q6_K and the 32-weight code
//   formats as exact bf16 codes with scales applied per group in fp32, Q5_K,
//   Q2_K, Q3_K and Q5_1 as fp32 weights split into bf16 hi + lo;
// * gemm_pw_kernel (M > 16; the same rows): 64 rows x 64 or 128 tokens per
//   workgroup, X tiles loaded straight into LDS, double-buffered; each wave
//   decodes its weight rows into bf16 hi/lo operands (two MFMAs per
//   product; one for the 32-weight code formats);
// * gemm_rows_kernel (the other shapes): one wave
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
// Few-token kernel (M <= 16, K-quants): exact-code MFMA products with W read
// straight from global memory, so that W streams once; only X passes
// through LDS.
//
// Slices. The MFMA's 16 weight columns (N) are R weight rows x 16/R slices
// of the super-block range, and its 16 token rows (M) are R tokens x the
// same 16/R slices: lane l holds the B operand of row (l % 16) % R in slice
// (l % 16) / R, and the A operand of token (l % 16) % R in the same slice,
// both at k-chunk l / 16. Output (t', n) then sums X[t' % R] against row
// n % R over slice n / R's columns wherever t' and n lie in the same slice
// (the other outputs mix slices and are dropped), and the epilogue adds
// the slices. A wave thereby covers R rows (R = 2, 4, 8 for M <= 2, 4, 8;
// 8 rows and two token sets for M <= 16) with the MFMA's full 16 x 16 x K
// operands, so a matrix of a few thousand rows still gives every CU
// workgroups, and no workgroup shares an output with another: no atomics,
// no zeroing launch, and the same result bits on every run.
//
// The KSW waves of a workgroup split the row's super-blocks; within a wave
// slice s takes super-blocks kb0 + S i + s (S = 16/R) at step i.
//
// Codes: a nibble or 6-bit code c becomes the bf16 value 128 + c with one
// v_perm_b32 per two codes (bits 0x43cc). A first MFMA multiplies the A
// operand by the constant -128 (Q4_K) or -160 (Q6_K: the offset 128 plus
// the code's -32), and feeds the product into the second one as its
// accumulator, which then holds sum X * c or sum X * (q - 32) over the
// group; the group's scale multiplies it in fp32:
//          Q4_K  acc += d*sc * P + (dmin*min / 128) * S   (S = -128 sum X)
//          Q6_K  acc += d*sc * P
// so no weight is ever rounded.
//
// Loads: a wave keeps D steps (W and X) in flight, in a ring of D register
// slots. All loads are raw buffer loads over the workgroup's R rows of W and
// over X; a slice past the wave's range gets an offset past the buffer, so
// its loads return zeros without reaching memory, with no branch around
// them (a load under a branch would make the compiler wait for every load
// at the join). Token rows past M and weight rows past the matrix read
// zeros the same way.
// ---------------------------------------------------------------------------

// A raw buffer over [base, base + bytes): loads at an offset past the end
// return zeros and reach no memory (the range check is on the per-lane
// offset, which therefore carries the whole offset; the scalar offset stays
// 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kPastEnd = 0x80000000u;  // an offset past every buffer here (the host keeps them < 2 GiB)
__device__ __forceinline__ u32x4 bld_b128(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, o, 0, 0);
}
__device__ __forceinline__ u32x2 bld_b64(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, o, 0, 0);
}
__device__ __forceinline__ uint32_t bld_b32(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, o, 0, 0);
}
__device__ __forceinline__ uint32_t bld_b16(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, o, 0, 0);
}

// bf16 pairs (128 + b0, 128 + b1) and (128 + b2, 128 + b3) of the four bytes of v
__device__ __forceinline__ uint32_t bf16_off_lo(uint32_t v) { return __builtin_amdgcn_perm(0x43434343u, v, 0x04010400u); }
__device__ __forceinline__ uint32_t bf16_off_hi(uint32_t v) { return __builtin_amdgcn_perm(0x43434343u, v, 0x04030402u); }

// ---------------------------------------------------------------------------
// Q5_K, Q2_K, Q3_K and Q5_1 on the matrix cores (both multi-token kernels).
// Each weight is formed in fp32 as the dequantiser forms it (the scale-and-
// offset step as one fused multiply-add: one rounding where the dequantiser
// rounds twice), then split into bf16 hi = w rounded to nearest even and
// lo = (w - hi) rounded the same way (w - hi is exact in fp32):
// |w - hi - lo| <= 2^-17 |w|, and the two products X * hi and X * lo
// accumulate in fp32, as Q4_K's operands do in the prefill kernel.
//
// HRaw<F>: the bytes lane (n, c) needs for 128 columns (half h of a
// super-block; for Q5_1 four 32-weight blocks), of whose chunk j (columns
// 32j .. 32j + 31) it holds columns 32j + 8c .. 32j + 8c + 7. Little-endian
// fields; layouts as in the dequantiser.
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
// 12 bytes from a 4-byte aligned address (one global_load_dwordx3).
__device__ __forceinline__ u32x3 ld_b96(const uint8_t *p) {
    u32x3 v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 12);
    return v;
}
__device__ __forceinline__ u32x3 bld_b96(__amdgpu_buffer_rsrc_t r, uint32_t o) {
    return __builtin_amdgcn_raw_buffer_load_b96(r, o, 0, 0);
}

template <int F> struct HRaw;
template <> struct HRaw<Q5_K> {
    u32x4 hd;    // d | dmin | packed 6-bit scales and mins (Q4_K's header)
    u32x2 q[2];  // nibble bytes 32g + 8c .. +7 of nibble groups g = 2h, 2h + 1
    u32x2 qh;    // fifth-bit bytes 8c .. 8c + 7
};
template <> struct HRaw<Q2_K> {
    u32x2 q;      // 2-bit code bytes 32h + 8c .. +7
    u32x2 s;      // scale | min bytes 8h .. 8h + 7 (one per 16 weights)
    uint32_t dd;  // d | dmin
};
template <> struct HRaw<Q3_K> {
    // 12-byte windows from the 4-byte boundary at or below the bytes (blocks
    // are 2-byte aligned); every window ends inside the block
    u32x3 hm;       // hmask bytes 8c .. 8c + 7
    u32x3 q;        // 2-bit code bytes 32h + 8c .. +7
    u32x3 s;        // packed scale bytes 0 .. 9 (from 96)
    uint32_t tail;  // block bytes 106 .. 109: scale bytes 10, 11 and d
    uint32_t mis;   // the block's offset from its 4-byte boundary (0 or 2)
};
template <> struct HRaw<Q5_1> {
    u32x2 dq[4];  // block j: d | m, then the fifth bits qh
    u32x2 q[4];   // block j: nibble bytes 8(c & 1) .. +7
};

__device__ __forceinline__ uint32_t byte_of(uint32_t w, int k) { return (w >> (8 * k)) & 0xFFu; }
__device__ __forceinline__ float byte_u(uint32_t w, int k) { return (float)byte_of(w, k); }

// bits 0..3 of n -> bit 4 of bytes 0..3
__device__ __forceinline__ uint32_t bit4_of_bytes(uint32_t n) { return (((n & 0xFu) * 0x00204081u) << 4) & 0x10101010u; }

// The lane's 8 weights of chunk j (h: the half; c: the lane's k chunk).
__device__ __forceinline__ void h_weights(const HRaw<Q5_K> &r, int h, int j, int, float w[8]) {
    const u32x4 hd = r.hd;
    const int sb = 4 * h + j;  // sub-block: scale, minimum and fifth-bit index
    const uint32_t SC = sb < 4 ? hd.y & 0x3F3F3F3Fu : (hd.w & 0x0F0F0F0Fu) | ((hd.y >> 2) & 0x30303030u);
    const uint32_t MN = sb < 4 ? hd.z & 0x3F3F3F3Fu : ((hd.w >> 4) & 0x0F0F0F0Fu) | ((hd.z >> 2) & 0x30303030u);
    const float dsc = half_bits_to_float(hd.x & 0xFFFFu) * byte_u(SC, j);
    const float m = half_bits_to_float(hd.x >> 16) * byte_u(MN, j);
    const u32x2 q = r.q[j >> 1];
    const int ns = 4 * (j & 1);
    const uint32_t c0 = ((q.x >> ns) & 0x0F0F0F0Fu) | (((r.qh.x >> sb) & 0x01010101u) << 4);
    const uint32_t c1 = ((q.y >> ns) & 0x0F0F0F0Fu) | (((r.qh.y >> sb) & 0x01010101u) << 4);
#pragma unroll
    for (int e = 0; e < 4; e++) {
        w[e] = __builtin_fmaf(dsc, byte_u(c0, e), -m);
        w[4 + e] = __builtin_fmaf(dsc, byte_u(c1, e), -m);
    }
}
__device__ __forceinline__ void h_weights(const HRaw<Q2_K> &r, int, int j, int c, float w[8]) {
    // scale | min byte 2j + c/2 of the half
    const uint32_t sb = byte_of(j < 2 ? r.s.x : r.s.y, (2 * j + (c >> 1)) & 3);
    const float dl = half_bits_to_float(r.dd & 0xFFFFu) * (float)(sb & 0xFu);
    const float ml = half_bits_to_float(r.dd >> 16) * (float)(sb >> 4);
    const uint32_t c0 = (r.q.x >> (2 * j)) & 0x03030303u, c1 = (r.q.y >> (2 * j)) & 0x03030303u;
#pragma unroll
    for (int e = 0; e < 4; e++) {
        w[e] = __builtin_fmaf(dl, byte_u(c0, e), -ml);
        w[4 + e] = __builtin_fmaf(dl, byte_u(c1, e), -ml);
    }
}
__device__ __forceinline__ void h_weights(const HRaw<Q3_K> &r, int h, int j, int c, float w[8]) {
    const uint32_t mis = r.mis;
    const uint32_t m0 = align_bytes(r.hm.y, r.hm.x, mis), m1 = align_bytes(r.hm.z, r.hm.y, mis);
    const uint32_t q0 = align_bytes(r.q.y, r.q.x, mis), q1 = align_bytes(r.q.z, r.q.y, mis);
    const uint32_t s0 = align_bytes(r.s.y, r.s.x, mis), s1 = align_bytes(r.s.z, r.s.y, mis);
    const uint32_t s2 = align_bytes(r.tail, r.s.z, mis);  // packed bytes 8 .. 11
    // scale si (one per 16 weights): low 4 bits in packed byte si (si < 8) or
    // the high nibble of byte si - 8, top 2 bits at bit 2 (si / 4) of byte
    // 8 + si % 4, stored + 32
    const int si = 8 * h + 2 * j + (c >> 1), k = si & 7;
    const uint32_t lb = byte_of(k < 4 ? s0 : s1, k & 3);
    const uint32_t lo4 = si < 8 ? lb & 0xFu : lb >> 4;
    const uint32_t hi2 = (s2 >> (8 * (si & 3) + 2 * (si >> 2))) & 3u;
    const float dsc = half_bits_to_float(r.tail >> 16) * (float)((int)(lo4 | (hi2 << 4)) - 32);
    // code + 4: the 2 bits, plus 4 where bit 4h + j of the hmask byte is set
    const int hb = 4 * h + j;
    const uint32_t u0 = ((q0 >> (2 * j)) & 0x03030303u) | (((m0 >> hb) & 0x01010101u) << 2);
    const uint32_t u1 = ((q1 >> (2 * j)) & 0x03030303u) | (((m1 >> hb) & 0x01010101u) << 2);
#pragma unroll
    for (int e = 0; e < 4; e++) {
        w[e] = dsc * (byte_u(u0, e) - 4.f);
        w[4 + e] = dsc * (byte_u(u1, e) - 4.f);
    }
}
__device__ __forceinline__ void h_weights(const HRaw<Q5_1> &r, int, int j, int c, float w[8]) {
    const u32x2 dq = r.dq[j], q = r.q[j];
    const float d = half_bits_to_float(dq.x & 0xFFFFu), m = half_bits_to_float(dq.x >> 16);
    const uint32_t hb = dq.y >> (8 * c);  // fifth bits of weights 8c .. 8c + 7
    const int ns = 4 * (c >> 1);          // weights 16 .. 31: the high nibbles
    const uint32_t c0 = ((q.x >> ns) & 0x0F0F0F0Fu) | bit4_of_bytes(hb);
    const uint32_t c1 = ((q.y >> ns) & 0x0F0F0F0Fu) | bit4_of_bytes(hb >> 4);
#pragma unroll
    for (int e = 0; e < 4; e++) {
        w[e] = __builtin_fmaf(byte_u(c0, e), d, m);
        w[4 + e] = __builtin_fmaf(byte_u(c1, e), d, m);
    }
}

// fp32 pair -> bf16 pair, each rounded to nearest even (v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2_v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_v){a, b}, bf16x2_v));
}

// The B operands (hi, lo) of eight fp32 weights.
__device__ __forceinline__ void split_rne8(const float w[8], u32x4 &bh, u32x4 &bl) {
    uint32_t hp[4], lp[4];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        const uint32_t hh = pk_bf16_rne(w[2 * e], w[2 * e + 1]);
        const float h0 = __builtin_bit_cast(float, hh << 16), h1 = __builtin_bit_cast(float, hh & 0xFFFF0000u);
        hp[e] = hh;
        lp[e] = pk_bf16_rne(w[2 * e] - h0, w[2 * e + 1] - h1);
    }
    bh = u32x4{hp[0], hp[1], hp[2], hp[3]};
    bl = u32x4{lp[0], lp[1], lp[2], lp[3]};
}

template <int F>
__device__ __forceinline__ void h_operands(const HRaw<F> &r, int h, int j, int c, u32x4 &bh, u32x4 &bl) {
    float w[8];
    h_weights(r, h, j, c, w);
    split_rne8(w, bh, bl);
}

template <int F> constexpr bool kHiLo = F == Q5_K || F == Q2_K || F == Q3_K || F == Q5_1;

template <int F> struct FewRaw;
template <> struct FewRaw<Q4_K> {
    u32x4 h;      // d | dmin | packed scales and mins
    u32x2 q[4];   // nibble bytes 32g + 8c .. +7 of the four nibble groups
};
template <> struct FewRaw<Q6_K> {
    u32x2 a[4], b[4], qh[4];  // per (h, lh): ql, ql + 32, qh windows (aligned down)
    u32x4 s;                  // scales (window)
    uint32_t t0, t1;          // bytes 206..207 (scales 14, 15) and 208..209 (d)
    uint32_t mis;             // the block's offset from its 4-byte boundary
};

// q8_0 and q4_0: the 8 blocks of a 256-column step; lane c holds codes
// 8c .. 8c + 7 of each (as in the prefill kernel)
template <> struct FewRaw<Q8_0> {
    uint32_t d[8];  // fp32 scales
    u32x2 q[8];     // codes 8c .. 8c + 7
};
template <> struct FewRaw<Q4_0> {
    uint32_t d[8];  // fp16 scales (low half)
    u32x2 q[8];     // nibble bytes 8(c & 1) .. +7, from the 4-byte boundary at or below them
    uint32_t t[4];  // even blocks (nibble bytes 2 past that boundary): their last two bytes
};
// GGUF's Q8_0 (34-byte blocks, fp16 d): as q4_0, an even block's codes sit
// 2 bytes past a 4-byte boundary, an odd block's on one
template <> struct FewRaw<Q8_0_F16> {
    uint32_t d[8];  // fp16 scales (low half)
    u32x2 q[8];     // code bytes 8c .. 8c + 7, from the 4-byte boundary at or below them
    uint32_t t[4];  // even blocks: their codes 8c + 6, 8c + 7
};

// Q5_K, Q2_K, Q3_K: one super-block; Q5_1: eight 32-weight blocks (as
// HRaw for each half, with what both halves share loaded once)
template <> struct FewRaw<Q5_K> {
    u32x4 hd;
    u32x2 q[4];  // nibble groups 0 .. 3
    u32x2 qh;
};
template <> struct FewRaw<Q2_K> {
    u32x2 q[2];  // per half
    u32x4 s;     // all 16 scale | min bytes
    uint32_t dd;
};
template <> struct FewRaw<Q3_K> {
    u32x3 hm, q[2], s;
    uint32_t t0, t1;  // bytes 106 .. 107 and 108 .. 109 (kept apart until use, as for Q6_K)
    uint32_t mis;
};
template <> struct FewRaw<Q5_1> {
    u32x2 dq[8], q[8];
};

__device__ __forceinline__ HRaw<Q5_K> few_half(const FewRaw<Q5_K> &r, int h) {
    return HRaw<Q5_K>{r.hd, {r.q[2 * h], r.q[2 * h + 1]}, r.qh};
}
__device__ __forceinline__ HRaw<Q2_K> few_half(const FewRaw<Q2_K> &r, int h) {
    return HRaw<Q2_K>{r.q[h], h ? u32x2{r.s.z, r.s.w} : u32x2{r.s.x, r.s.y}, r.dd};
}
__device__ __forceinline__ HRaw<Q3_K> few_half(const FewRaw<Q3_K> &r, int h) {
    return HRaw<Q3_K>{r.hm, r.q[h], r.s, r.t0 | (r.t1 << 16), r.mis};
}
__device__ __forceinline__ HRaw<Q5_1> few_half(const FewRaw<Q5_1> &r, int h) {
    HRaw<Q5_1> v;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        v.dq[j] = r.dq[4 * h + j];
        v.q[j] = r.q[4 * h + j];
    }
    return v;
}

// X reaches the MFMA through wave-private LDS tiles of S * TM rows (slice s,
// token t < TM at row s TM + t; one tile per token set) x 256 columns (one
// super-block per slice; rows padded by 16 bytes): lane l loads 16-byte
// chunk l % 32 of tile rows l / 32, 2 + l / 32, ... (coalesced along the
// row), stores them to the tile, and reads its A operands from the row of
// its slice and token, or of token t % TM where t >= TM: those results
// belong to tokens past M and are not stored, so a tile holds only the
// tokens below M (TM, the power of two at or above M, up to R). Read
// straight from X by each lane for its own token, the token rows of one
// load instruction sit ldx apart (4 KiB at 2048 columns) and fall on the
// same L1 cache sets; the tag conflicts stalled the address pipeline.
constexpr int FEW_LX = 264;  // bf16 per tile row

// o: the block's byte offset in the W buffer (or kPastEnd)
template <int F>
__device__ __forceinline__ void few_load(FewRaw<F> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c);

template <>
__device__ __forceinline__ void few_load<Q4_K>(FewRaw<Q4_K> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c) {
    r.h = bld_b128(wr, o);
#pragma unroll
    for (int g = 0; g < 4; g++) r.q[g] = bld_b64(wr, o + 16 + 32 * g + 8 * c);
}

template <>
__device__ __forceinline__ void few_load<Q6_K>(FewRaw<Q6_K> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c) {
    const uint32_t a0 = o & ~3u;  // 4-byte aligned (the buffer's base is); blocks are 2-byte aligned
    r.mis = o & 3u;
#pragma unroll
    for (int hl = 0; hl < 4; hl++) {
        const int h = hl >> 1, lh = hl & 1;
        r.a[hl] = bld_b64(wr, a0 + 64 * h + 16 * lh + 4 * c);
        r.b[hl] = bld_b64(wr, a0 + 64 * h + 32 + 16 * lh + 4 * c);
        r.qh[hl] = bld_b64(wr, a0 + 128 + 32 * h + 16 * lh + 4 * c);
    }
    r.s = bld_b128(wr, a0 + 192);
    // (kept apart until the multiply: combined here, the two values would
    // make the wave wait for every load issued before them)
    r.t0 = bld_b16(wr, o + 206);
    r.t1 = bld_b16(wr, o + 208);
}

// o: the step's first block (4-byte aligned: row bytes are multiples of 144
// when the columns are a multiple of 256); even blocks' nibble bytes sit 2
// bytes past a 4-byte boundary, odd blocks' on one
template <>
__device__ __forceinline__ void few_load<Q8_0>(FewRaw<Q8_0> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
        r.d[j] = bld_b32(wr, o + 36 * j);
        r.q[j] = bld_b64(wr, o + 36 * j + 4 + 8 * c);
    }
}
template <>
__device__ __forceinline__ void few_load<Q4_0>(FewRaw<Q4_0> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t q = o + 18 * j + 2 + 8 * (c & 1);
        r.d[j] = bld_b16(wr, o + 18 * j);
        if (j % 2 == 0) {
            r.q[j] = bld_b64(wr, q - 2);
            r.t[j / 2] = bld_b16(wr, q + 6);
        } else {
            r.q[j] = bld_b64(wr, q);
        }
    }
}

template <>
__device__ __forceinline__ void few_load<Q8_0_F16>(FewRaw<Q8_0_F16> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o,
                                                   int c) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
        const uint32_t q = o + 34 * j + 2 + 8 * c;
        r.d[j] = bld_b16(wr, o + 34 * j);
        if (j % 2 == 0) {
            r.q[j] = bld_b64(wr, q - 2);
            r.t[j / 2] = bld_b16(wr, q + 6);
        } else {
            r.q[j] = bld_b64(wr, q);
        }
    }
}

template <>
__device__ __forceinline__ void few_load<Q5_K>(FewRaw<Q5_K> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c) {
    r.hd = bld_b128(wr, o);
    r.qh = bld_b64(wr, o + 16 + 8 * c);
#pragma unroll
    for (int g = 0; g < 4; g++) r.q[g] = bld_b64(wr, o + 48 + 32 * g + 8 * c);
}
template <>
__device__ __forceinline__ void few_load<Q2_K>(FewRaw<Q2_K> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c) {
    r.s = bld_b128(wr, o);
#pragma unroll
    for (int h = 0; h < 2; h++) r.q[h] = bld_b64(wr, o + 16 + 32 * h + 8 * c);
    r.dd = bld_b32(wr, o + 80);
}
template <>
__device__ __forceinline__ void few_load<Q3_K>(FewRaw<Q3_K> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c) {
    const uint32_t a0 = o & ~3u;  // 4-byte aligned (the buffer's base is); blocks are 2-byte aligned
    r.mis = o & 3u;
    r.hm = bld_b96(wr, a0 + 8 * c);
#pragma unroll
    for (int h = 0; h < 2; h++) r.q[h] = bld_b96(wr, a0 + 32 + 32 * h + 8 * c);
    r.s = bld_b96(wr, a0 + 96);
    r.t0 = bld_b16(wr, o + 106);
    r.t1 = bld_b16(wr, o + 108);
}
// o: the step's first block (8-byte aligned: 24-byte blocks, rows of whole
// 192-byte steps)
template <>
__device__ __forceinline__ void few_load<Q5_1>(FewRaw<Q5_1> &r, __amdgpu_buffer_rsrc_t wr, uint32_t o, int c) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
        r.dq[j] = bld_b64(wr, o + 24 * j);
        r.q[j] = bld_b64(wr, o + 24 * j + 8 + 8 * (c & 1));
    }
}

// q8_0 codes as bf16 (exact: integers of at most 8 bits); q4_0 codes as
// bf16 128 + n from the nibble bytes, realigned for even blocks
__device__ __forceinline__ u32x4 codes_q8_0(u32x2 q) {
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        f[e] = (float)(int)(int8_t)(q.x >> (8 * e));
        f[4 + e] = (float)(int)(int8_t)(q.y >> (8 * e));
    }
    auto top2 = [](float lo, float hi) {
        return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
    };
    return u32x4{top2(f[0], f[1]), top2(f[2], f[3]), top2(f[4], f[5]), top2(f[6], f[7])};
}
__device__ __forceinline__ u32x4 codes_q4_0(u32x2 q, uint32_t tail, bool realign, int c) {
    const uint32_t w0 = realign ? align_bytes(q.y, q.x, 2) : q.x;
    const uint32_t w1 = realign ? align_bytes(tail, q.y, 2) : q.y;
    const int sh = 4 * (c >> 1);
    const uint32_t n0 = (w0 >> sh) & 0x0F0F0F0Fu, n1 = (w1 >> sh) & 0x0F0F0F0Fu;
    return u32x4{bf16_off_lo(n0), bf16_off_hi(n0), bf16_off_lo(n1), bf16_off_hi(n1)};
}

// xa: this lane's row of the first X tile, offset to its k chunk c = lane /
// 16 (8 columns of the chunk for Q4_K, 4 for Q6_K); the tile of token set
// ts follows at ts * XT bf16. Groups go four at a time: the four products
// against the constant first, then the four against the codes (each fed
// the first as its accumulator), so that no product waits for the one just
// issued.
template <int TS, int XT>
__device__ __forceinline__ void few_mma_q4k(const FewRaw<Q4_K> &r, const uint16_t *xa, f32x4 (&acc)[TS]) {
    const u32x4 h = r.h;
    const float d = half_bits_to_float(h.x & 0xFFFFu);
    const float dmin = half_bits_to_float(h.x >> 16) * (1.0f / 128.0f);  // exact: a power of two
    const uint32_t sc_lo = h.y & 0x3F3F3F3Fu, mn_lo = h.z & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t mn_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    const u32x4 m128 = u32x4{0xC300C300u, 0xC300C300u, 0xC300C300u, 0xC300C300u};  // bf16 -128
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += 4) {
        const uint32_t SC = j0 == 0 ? sc_lo : sc_hi, MN = j0 == 0 ? mn_lo : mn_hi;
        float dsc[4], dmn[4];
        u32x4 bw[4];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int j = j0 + jj;
            dsc[jj] = d * (float)((SC >> (8 * jj)) & 0xFFu);
            dmn[jj] = dmin * (float)((MN >> (8 * jj)) & 0xFFu);
            const u32x2 q = r.q[j >> 1];
            const uint32_t n0 = (j & 1) ? (q.x >> 4) & 0x0F0F0F0Fu : q.x & 0x0F0F0F0Fu;
            const uint32_t n1 = (j & 1) ? (q.y >> 4) & 0x0F0F0F0Fu : q.y & 0x0F0F0F0Fu;
            bw[jj] = u32x4{bf16_off_lo(n0), bf16_off_hi(n0), bf16_off_lo(n1), bf16_off_hi(n1)};
        }
#pragma unroll
        for (int ts = 0; ts < TS; ts++) {
            bf16x8 av[4];
            f32x4 S[4], P[4];
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                // X[t][32j + 8c .. +7]
                av[jj] = *reinterpret_cast<const bf16x8 *>(xa + ts * XT + 32 * (j0 + jj));
                S[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[jj], __builtin_bit_cast(bf16x8, m128),
                                                               f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int jj = 0; jj < 4; jj++)
                P[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[jj], __builtin_bit_cast(bf16x8, bw[jj]), S[jj], 0,
                                                               0, 0);
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                acc[ts] += dsc[jj] * P[jj];
                acc[ts] += dmn[jj] * S[jj];
            }
        }
    }
}

template <int TS, int XT>
__device__ __forceinline__ void few_mma_q6k(const FewRaw<Q6_K> &r, const uint16_t *xa, f32x4 (&acc)[TS]) {
    const uint32_t mis = r.mis;
    const uint32_t s4 = r.t0 | (r.t1 << 16);  // bytes 206..209
    const uint32_t s0 = align_bytes(r.s.y, r.s.x, mis), s1 = align_bytes(r.s.z, r.s.y, mis);
    const uint32_t s2 = align_bytes(r.s.w, r.s.z, mis), s3 = align_bytes(s4, r.s.w, mis);
    const uint32_t sw[4] = {s0, s1, s2, s3};  // scales 0..15
    const float d = half_bits_to_float(r.t1);
    const u32x2 m160 = u32x2{0xC320C320u, 0xC320C320u};  // bf16 -160
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
        float dsc[4];
        u32x2 bw[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int gi = 8 * h + 2 * k + lh;
            dsc[k] = d * (float)(int)(int8_t)(sw[gi >> 2] >> (8 * (gi & 3)));
            bw[k] = u32x2{bf16_off_lo(code[k]), bf16_off_hi(code[k])};
        }
#pragma unroll
        for (int ts = 0; ts < TS; ts++) {
            s16x4 av[4];
            f32x4 S[4], P[4];
#pragma unroll
            for (int k = 0; k < 4; k++) {
                // X[t][16 gi + 4c .. +3]
                av[k] = *reinterpret_cast<const s16x4 *>(xa + ts * XT + 16 * (8 * h + 2 * k + lh));
                S[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[k], __builtin_bit_cast(s16x4, m160),
                                                                f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int k = 0; k < 4; k++)
                P[k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av[k], __builtin_bit_cast(s16x4, bw[k]), S[k], 0, 0,
                                                                0);
#pragma unroll
            for (int k = 0; k < 4; k++) acc[ts] += dsc[k] * P[k];
        }
    }
}

// q8_0 / q4_0: one product per block (a 16x16x32 chunk), scaled by the
// block's d; q4_0's offset product (X against -136 = -(128 + 8)) is the code
// product's accumulator. Blocks go four at a time, as above.
template <int F, int TS, int XT>
__device__ __forceinline__ void few_mma_b32(const FewRaw<F> &r, const uint16_t *xa, f32x4 (&acc)[TS], int c) {
    const u32x4 m136 = u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};  // bf16 -136
#pragma unroll
    for (int j0 = 0; j0 < 8; j0 += 4) {
        u32x4 bw[4];
        float d[4];
#pragma unroll
        for (int jj = 0; jj < 4; jj++) {
            const int j = j0 + jj;
            if constexpr (F == Q8_0) {
                bw[jj] = codes_q8_0(r.q[j]);
                d[jj] = __builtin_bit_cast(float, r.d[j]);
            } else if constexpr (F == Q8_0_F16) {
                u32x2 q = r.q[j];
                if (j % 2 == 0) q = u32x2{align_bytes(q.y, q.x, 2), align_bytes(r.t[j / 2], q.y, 2)};  // realign
                bw[jj] = codes_q8_0(q);
                d[jj] = half_bits_to_float(r.d[j] & 0xFFFFu);
            } else {
                bw[jj] = codes_q4_0(r.q[j], r.t[j / 2], j % 2 == 0, c);
                d[jj] = half_bits_to_float(r.d[j] & 0xFFFFu);
            }
        }
#pragma unroll
        for (int ts = 0; ts < TS; ts++) {
            bf16x8 av[4];
            f32x4 P[4];
#pragma unroll
            for (int jj = 0; jj < 4; jj++) {
                av[jj] = *reinterpret_cast<const bf16x8 *>(xa + ts * XT + 32 * (j0 + jj));  // X[t][32j + 8c .. +7]
                P[jj] = F == Q4_0 ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[jj], __builtin_bit_cast(bf16x8, m136),
                                                                           f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)
                                  : f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int jj = 0; jj < 4; jj++)
                P[jj] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[jj], __builtin_bit_cast(bf16x8, bw[jj]), P[jj], 0, 0,
                                                               0);
#pragma unroll
            for (int jj = 0; jj < 4; jj++) acc[ts] += d[jj] * P[jj];
        }
    }
}

// Q5_K, Q2_K, Q3_K, Q5_1: two products per chunk (X * hi, then X * lo into
// it), four chunks at a time, added into the accumulators.
template <int F, int TS, int XT>
__device__ __forceinline__ void few_mma_hl(const FewRaw<F> &r, const uint16_t *xa, f32x4 (&acc)[TS], int c) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const HRaw<F> hr = few_half(r, h);
        u32x4 bh[4], bl[4];
#pragma unroll
        for (int j = 0; j < 4; j++) h_operands<F>(hr, h, j, c, bh[j], bl[j]);
#pragma unroll
        for (int ts = 0; ts < TS; ts++) {
            bf16x8 av[4];
            f32x4 P[4];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                av[j] = *reinterpret_cast<const bf16x8 *>(xa + ts * XT + 32 * (4 * h + j));  // X[t][32j' + 8c .. +7]
                P[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], __builtin_bit_cast(bf16x8, bh[j]),
                                                              f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            }
#pragma unroll
            for (int j = 0; j < 4; j++)
                P[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[j], __builtin_bit_cast(bf16x8, bl[j]), P[j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < 4; j++) acc[ts] += P[j];
        }
    }
}

template <int F, int TS, int XT>
__device__ __forceinline__ void few_mma(const FewRaw<F> &r, const uint16_t *xa, f32x4 (&acc)[TS], int c) {
    if constexpr (F == Q4_K)
        few_mma_q4k<TS, XT>(r, xa, acc);
    else if constexpr (F == Q6_K)
        few_mma_q6k<TS, XT>(r, xa, acc);
    else if constexpr (kHiLo<F>)
        few_mma_hl<F, TS, XT>(r, xa, acc, c);
    else
        few_mma_b32<F, TS, XT>(r, xa, acc, c);
}

// R rows per wave and workgroup, TM tokens per slice in the X tile, TS token
// sets of 8 (TS = 2 only with R = TM = 8), D steps in flight
template <int F, int R, int TM, int TS, int D>
__global__ __launch_bounds__(512) void gemm_few_kernel(const uint8_t *W, int rows, int nb, int64_t row_bytes,
                                                       const uint16_t *X, int M, float *Y) {
    static_assert(R == 8 || R == 16, "rows per wave");
    static_assert(TM >= 1 && TM <= R && (TM & (TM - 1)) == 0, "tokens per slice in the tile");
    static_assert(TS == 1 || (R == 8 && TM == 8), "two token sets of 8");
    constexpr int BYTES = Layout<F>::BYTES * (256 / Layout<F>::QK);  // per 256 columns
    constexpr int S = 16 / R;        // slices
    constexpr int TR = S * TM;       // tile rows (>= 2)
    constexpr int NJ = TR / 2;       // 16-byte loads per lane and tile
    constexpr int XT = TR * FEW_LX;  // bf16 per tile
    // per wave: its tiles, whose space also takes its partial results at the end
    constexpr int WAVE_LDS = (TS * XT * 2 > TS * 1024 ? TS * XT * 2 : TS * 1024) / 2;  // bf16
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int ksw = blockDim.x >> 6;
    const int n = lane & 15, c = lane >> 4;
    // W: the workgroup's R rows (fewer in the last one), from the 4-byte
    // boundary at or below their first byte; this lane's row n % R in
    // slice n / R
    const int row0 = (int)blockIdx.x * R;
    const uint8_t *const tile = W + (int64_t)row0 * row_bytes;
    const uint32_t mis0 = (uint32_t)(uintptr_t)tile & 3u;
    const __amdgpu_buffer_rsrc_t wr = raw_rsrc(tile - mis0, (uint32_t)(min(R, rows - row0) * row_bytes) + mis0);
    const uint32_t wlane = (uint32_t)((n % R) * row_bytes) + mis0;
    const int wslice = n / R;
    // X: M token rows of nb * 512 bytes
    const uint32_t xrow = (uint32_t)nb * 512u;
    const __amdgpu_buffer_rsrc_t xr = raw_rsrc(X, (uint32_t)M * xrow);
    extern __shared__ __attribute__((aligned(16))) uint16_t few_xs[];
    uint16_t *const xw = few_xs + wave * WAVE_LDS;  // this wave's X tiles
    // its A operands: k chunk c is 8 columns wide for the 16x16x32 product
    // (Q4_K, q8_0, q4_0), 4 for the 16x16x16 one (Q6_K)
    const uint16_t *const xa = xw + (wslice * TM + (n % R) % TM) * FEW_LX + (F == Q6_K ? 4 : 8) * c;
    // this wave's part of the super-blocks [kb0, kb0 + cnt), spread evenly
    // (every wave has at least one: the host keeps ksw <= nb)
    const int kb0 = wave * nb / ksw, cnt = (wave + 1) * nb / ksw - kb0;
    const int steps = (cnt + S - 1) / S;

    f32x4 acc[TS];
#pragma unroll
    for (int ts = 0; ts < TS; ts++) acc[ts] = f32x4{0.f, 0.f, 0.f, 0.f};
    FewRaw<F> buf[D];
    u32x4 xb[D][TS][NJ];
    // slot sl <- step i (zeros past the wave's range); tile row tr = 2j +
    // lane / 32 holds token tr % TM (+ 8 ts) of slice tr / TM
    auto issue = [&](int sl, int i) {
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const int tr = 2 * j + (lane >> 5), k = i * S + tr / TM;
#pragma unroll
            for (int ts = 0; ts < TS; ts++) {
                const uint32_t o = (uint32_t)(8 * ts + tr % TM) * xrow + (uint32_t)(kb0 + k) * 512u +
                                   16u * (uint32_t)(lane & 31);
                xb[sl][ts][j] = bld_b128(xr, k < cnt ? o : kPastEnd);
            }
        }
        const int k = i * S + wslice;
        few_load<F>(buf[sl], wr, k < cnt ? wlane + (uint32_t)(kb0 + k) * (uint32_t)BYTES : kPastEnd, c);
    };
    auto xstore = [&](int sl) {
#pragma unroll
        for (int ts = 0; ts < TS; ts++)
#pragma unroll
            for (int j = 0; j < NJ; j++)
                *reinterpret_cast<u32x4 *>(xw + ts * XT + (2 * j + (lane >> 5)) * FEW_LX + 8 * (lane & 31)) =
                    xb[sl][ts][j];
    };
    // The loop starts D steps early: its first round only fills the slots
    // (its tile stores write nothing that is read), so that the loads
    // before the loop are issued by the same code, in the same order, as
    // those inside it, and the waits the compiler places at the top of the
    // loop hold for every round.
#pragma unroll
    for (int sl = 0; sl < D; sl++)
#pragma unroll
        for (int ts = 0; ts < TS; ts++)
#pragma unroll
            for (int j = 0; j < NJ; j++) xb[sl][ts][j] = u32x4{0u, 0u, 0u, 0u};
    for (int i0 = -D; i0 < steps; i0 += D) {
#pragma unroll
        for (int sl = 0; sl < D; sl++) {
            // the slot's X tiles replace the last ones after their multiplies
            // (the LDS accesses of a wave stay in order), then the slot is
            // refilled D steps ahead
            xstore(sl);
            if (i0 >= 0 && i0 + sl < steps) few_mma<F, TS, XT>(buf[sl], xa, acc, c);
            issue(sl, i0 + sl + D);
            // (the empty asm keeps earlier passes from moving loads across
            // slots, the scheduling barrier the scheduler)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    // lane (n, c) holds outputs t' = 4c + i of column n; (t', n) counts where
    // both lie in one slice: token t' % R of row n % R. Each wave leaves its
    // partial tiles in its own LDS space (after its last reads of it: the
    // LDS accesses of a wave stay in order); they are added over the waves,
    // then the slices, in a fixed order.
    f32x4 *const part = reinterpret_cast<f32x4 *>(few_xs);
    constexpr int PW = WAVE_LDS / 8;  // f32x4 per wave
#pragma unroll
    for (int ts = 0; ts < TS; ts++) part[wave * PW + ts * 64 + lane] = acc[ts];
    __syncthreads();
    // (TS * R * R <= 128 outputs; a workgroup of one wave takes two rounds)
    for (int o = threadIdx.x; o < TS * R * R; o += blockDim.x) {
        const int ts = o / (R * R), t = (o / R) % R, rr = o % R;
        float sum = 0.f;
        for (int w = 0; w < ksw; w++)
#pragma unroll
            for (int sl = 0; sl < S; sl++) {
                const int tp = sl * R + t;
                sum += part[w * PW + ts * 64 + 16 * (tp >> 2) + sl * R + rr][tp & 3];
            }
        const int m = 8 * ts + t, row = row0 + rr;
        if (m < M && row < rows) Y[(int64_t)m * rows + row] = sum;
    }
}

// Waves per workgroup and steps of loads in flight at M <= 8, from the
// workgroups (row tiles of 8) per CU: above 2.5 one wave (two steps in
// flight at M <= 2 or below 4 workgroups per CU, else one); from 1.5 to 2.5
// four waves on rows of 16 or more super-blocks, else two (two steps at M <=
// 2, else one). At 1.5 and below, rows of 13 or more super-blocks take about
// 3 waves per CU (2 where the super-blocks are a power of two, so that they
// split evenly) with two steps; shorter rows about 4 waves per CU, each with
// at least two super-blocks, and one step. Swept over 1, 2, 3, 4 waves x 1,
// 2 steps at M = 1, 2, 4, 8 on 18 shapes (Q4_K 5632 x 2048, 2048 x 2048,
// 4096 x 4096, 11008 x 4096, 1024 x 1024, 1024 x 4096, 2304 x 2304, 3072 x
// 3072; Q6_K 2048 x 5632, 4096 x 11008, 32000 x 2048, 2048 x 2048, 1536 x
// 2048, 2560 x 2560, 3072 x 3072; q8_0 5632 x 2048, 3584 x 3584; q4_0 5632 x
// 2048): within 1.0 % of the fastest on average and 13 % at worst (the rule
// before, with about 3 waves per CU and two steps for every row length at
// 1.5 and below: 4.7 % and 25 %; 2560 x 2560 Q6_K at M = 8 9.3 -> 7.8 us).
inline int64_t few_waves(int64_t wgs, int64_t nb) {
    const double wpc = (double)wgs / (double)device_cu_count();
    if (wpc > 2.5) return 1;
    if (wpc > 1.5) return nb >= 16 ? 4 : 2;
    if (nb <= 12) {
        int64_t k = (int64_t)(4.0 / wpc + 0.5);
        if (k > nb / 2) k = nb / 2;
        return k < 1 ? 1 : k;
    }
    int64_t k = (int64_t)(3.0 / wpc + 0.5);
    if (k < 1) k = 1;
    if (k == 3 && (nb & (nb - 1)) == 0) k = 2;
    return k;
}
inline int few_depth(int64_t rows, int64_t nb, int64_t M) {
    if (M > 8) return 1;
    const double wpc = (double)((rows + 7) / 8) / (double)device_cu_count();
    if (wpc > 2.5) return M <= 2 || wpc < 4 ? 2 : 1;
    if (wpc > 1.5) return M <= 2 ? 2 : 1;
    return nb <= 12 ? 1 : 2;
}

template <int F, int R, int TM, int TS, int D>
static hipError_t launch_few_r(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                               int64_t M, float *Y, hipStream_t stream) {
    constexpr int TR = (16 / R) * TM, XT = TR * FEW_LX;
    constexpr int WAVE_BYTES = TS * XT * 2 > TS * 1024 ? TS * XT * 2 : TS * 1024;
    const int nb = (int)(cols / 256);
    const int64_t wgs = (rows + R - 1) / R;
    // waves per workgroup, at most 4 and no more than one per super-block;
    // QK_TUNE_FEW_KSW sets it (1..8). M <= 8: few_waves (below); M > 8:
    // about 4 waves per CU, where each wave carries twice the products.
    const int64_t cus = device_cu_count();
    int64_t ksw = M <= 8 ? few_waves(wgs, nb) : (4 * cus + wgs - 1) / wgs;
    if (ksw > 4) ksw = 4;
    if (tuning(QK_TUNE_FEW_KSW) > 0) ksw = tuning(QK_TUNE_FEW_KSW);
    if (ksw > 8) ksw = 8;
    if (ksw > nb) ksw = nb;
    if (ksw < 1) ksw = 1;
    const size_t shmem = (size_t)ksw * WAVE_BYTES;  // the waves' X tiles
    if (shmem > 49152) {
        // more than the default dynamic LDS (set once per device)
        const hipError_t e = allow_max_dynamic_lds(reinterpret_cast<const void *>(gemm_few_kernel<F, R, TM, TS, D>));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((gemm_few_kernel<F, R, TM, TS, D>), dim3((unsigned)wgs), dim3((unsigned)(64 * ksw)), shmem,
                       stream, W, (int)rows, nb, row_bytes, X, (int)M, Y);
    return hipGetLastError();
}

template <int F, int D>
static hipError_t launch_few_d(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                               int64_t M, float *Y, hipStream_t stream) {
    if (M <= 8) {
        if (M == 1) return launch_few_r<F, 8, 1, 1, D>(W, rows, cols, row_bytes, X, M, Y, stream);
        if (M == 2) return launch_few_r<F, 8, 2, 1, D>(W, rows, cols, row_bytes, X, M, Y, stream);
        if (M <= 4) return launch_few_r<F, 8, 4, 1, D>(W, rows, cols, row_bytes, X, M, Y, stream);
        return launch_few_r<F, 8, 8, 1, D>(W, rows, cols, row_bytes, X, M, Y, stream);
    }
    // M > 8: 8 rows in two slices with two token sets where the 8-row
    // workgroups fit the CUs in one round, else 16 rows of one slice; Q4_K
    // always 16. Swept at M = 12 and 16 over 1024-32000 rows of every
    // format: 2048 x 5632 Q6_K 9.6 (8 rows) against 12.0 us (16), 2048 x 2048
    // q8_0 6.1 against 7.5; from 2304 rows on, 16 rows won by 5-33 % (3584 x
    // 3584 Q6_K 9.6 against 11.9 us, 2816 x 2048 Q4_K 5.1 against 7.5), and
    // for Q4_K also at 1024 and 2048 rows (2048 x 2048 5.0 against 5.4).
    // QK_TUNE_FEW_ROWS = 8 or 16 sets it.
    const int rf = tuning(QK_TUNE_FEW_ROWS);
    const bool r16 = rf == 16 || (rf != 8 && (F == Q4_K || rows > (int64_t)8 * device_cu_count()));
    if (r16) return launch_few_r<F, 16, 16, 1, D>(W, rows, cols, row_bytes, X, M, Y, stream);
    return launch_few_r<F, 8, 8, 2, D>(W, rows, cols, row_bytes, X, M, Y, stream);
}

// Steps of loads in flight: few_depth above at M <= 8, one above M = 8
// (measured at M = 12 and 16: the second slot's registers cost more
// occupancy than it gains once the X tiles grow); QK_TUNE_FEW_DEPTH = 1 or
// 2 sets it.
template <int F>
static hipError_t launch_few(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                             int64_t M, float *Y, hipStream_t stream) {
    const int df = tuning(QK_TUNE_FEW_DEPTH);
    const int depth = df == 1 || df == 2 ? df : few_depth(rows, cols / 256, M);
    if (depth == 2) return launch_few_d<F, 2>(W, rows, cols, row_bytes, X, M, Y, stream);
    return launch_few_d<F, 1>(W, rows, cols, row_bytes, X, M, Y, stream);
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
// Prefill kernel (M > 16: every format).
//
// A workgroup computes 64 weight rows x TOK tokens (TOK = 64 or 128); each
// of its 4 waves owns 16 rows and all TOK tokens (TOK / 16 M tiles of
// v_mfma_f32_16x16x32_bf16), so every weight a wave decodes feeds TOK / 16
// products. K advances 128 columns (half a super-block) per step. The step's
// TOK x 128 bf16 X tile goes straight from global memory to LDS with 16-byte
// direct loads (no registers on the way) into one of two buffers, one step
// ahead; the weights are loaded into registers two steps ahead. The tile is
// unpadded: 16-byte chunk k of token m sits at slot k ^ (m % 16) of the
// token's 256 bytes, so the 16 lanes that read one chunk column of 16
// tokens hit 16 different bank groups.
//
// Operands (two MFMAs per product, X * hi + X * lo, fp32 accumulation):
//   Q6_K  v = sc * (q - 32), an integer of at most 13 bits, split exactly
//         into bf16 v_hi + v_lo; every product is exact and the super-block's
//         d multiplies the sums of its two steps;
//   Q4_K  w = (d*sc)*q - dmin*mn in fp32 (one rounding), split into
//         w_hi = w rounded to bf16 (nearest even) and w_lo = (w - w_hi)
//         rounded to bf16 (w - w_hi is exact in fp32):
//         |w - w_hi - w_lo| <= 2^-17 |w|, so the result stays within
//         2^-17 * sum|w*x| of the exact products' sum (plus the fp32
//         accumulation), far inside the tolerance for any input; the
//         minimum term needs no third MFMA;
//   q8_0  codes as exact bf16, one MFMA per 32-weight block and M tile,
//         scaled by the block's d; q4_0 the same with codes 128 + n and the
//         -136 offset product as the accumulator; GGUF's Q8_0 as q8_0;
//   Q5_K, Q2_K, Q3_K, Q5_1  as Q4_K (h_operands).
//
// KH = 2 splits K over two workgroups (blockIdx.z) that add their sums
// into Y, which a fill launch zeroes first (two addends to zero: the order
// does not change the result); used where the row and token tiles alone
// leave CUs idle (the 2048 x 5632 down shape).
// ---------------------------------------------------------------------------

// Raw bytes of one half super-block for lane (n, c).
template <int F> struct PwRaw;
template <> struct PwRaw<Q4_K> {
    u32x4 h;     // d | dmin | packed scales and mins
    u32x2 q[2];  // nibble bytes 32g + 8c .. +7 of the half's two nibble groups
};
template <> struct PwRaw<Q6_K> {
    // (12-byte windows: the decode uses three dwords of each; a fourth,
    // loaded and never read, would have its register reused while the load
    // is in flight, which makes the wave wait for every load)
    u32x3 ql[2];  // ql windows 64h + 32p + 8c (p = 0, 1), from the 4-byte boundary below
    u32x3 qh;     // qh window 128 + 32h + 8c
    u32x4 s;      // scales window
    uint32_t s4;  // q6k_tail: scales 14, 15 and d
    uint32_t mis; // bytes from the 4-byte boundary below the block to it (0 or 2)
};

__device__ __forceinline__ void pw_load(PwRaw<Q4_K> &r, const uint8_t *blk, int h, int c) {
    r.h = ld_b128(blk);
#pragma unroll
    for (int i = 0; i < 2; i++) r.q[i] = ld_b64(blk + 16 + 32 * (2 * h + i) + 8 * c);
}

// (every window stays inside the block: the last ql window ends at byte 132
// of the aligned-down block, the qh windows at 196, the scales at 208)
__device__ __forceinline__ void pw_load(PwRaw<Q6_K> &r, const uint8_t *blk, int h, int c) {
    r.mis = (uint32_t)(uintptr_t)blk & 3u;
    const uint8_t *A0 = blk - r.mis;
#pragma unroll
    for (int p = 0; p < 2; p++) r.ql[p] = ld_b96(A0 + 64 * h + 32 * p + 8 * c);
    r.qh = ld_b96(A0 + 128 + 32 * h + 8 * c);
    r.s = ld_b128(A0 + 192);
    r.s4 = q6k_tail(blk);
}

// B operands (hi, lo) of chunk j (columns 32j.. of half h) for lane c.
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
    uint32_t hp[4], lp[4];
#pragma unroll
    for (int k = 0; k < 2; k++) {
        const uint32_t nn = k ? n1 : n0;
        const auto p0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)nn, false);
        const auto p1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)nn, true);
        const float w[4] = {__builtin_fmaf(a, p0[0], -b), __builtin_fmaf(a, p0[1], -b), __builtin_fmaf(a, p1[0], -b),
                            __builtin_fmaf(a, p1[1], -b)};
#pragma unroll
        for (int e = 0; e < 2; e++) {
            const uint32_t hh = pk_bf16_rne(w[2 * e], w[2 * e + 1]);
            const float h0 = __builtin_bit_cast(float, hh << 16), h1 = __builtin_bit_cast(float, hh & 0xFFFF0000u);
            hp[2 * k + e] = hh;
            lp[2 * k + e] = pk_bf16_rne(w[2 * e] - h0, w[2 * e + 1] - h1);
        }
    }
    bh = u32x4{hp[0], hp[1], hp[2], hp[3]};
    bl = u32x4{lp[0], lp[1], lp[2], lp[3]};
}

__device__ __forceinline__ void pw_dec(const PwRaw<Q6_K> &r, int h, int j, int c, u32x4 &bh, u32x4 &bl) {
    const uint32_t mis = r.mis;
    // quarter j of half h: ql window p = j & 1 (low nibbles for j < 2), qh bits 2j
    const u32x3 A = r.ql[j & 1], H = r.qh;
    const uint32_t a0 = align_bytes(A.y, A.x, mis), a1 = align_bytes(A.z, A.y, mis);
    const uint32_t h0 = align_bytes(H.y, H.x, mis), h1 = align_bytes(H.z, H.y, mis);
    const int ns = j >= 2 ? 4 : 0;
    const uint32_t q0 = ((a0 >> ns) & 0x0F0F0F0Fu) | (((h0 >> (2 * j)) & 0x03030303u) << 4);
    const uint32_t q1 = ((a1 >> ns) & 0x0F0F0F0Fu) | (((h1 >> (2 * j)) & 0x03030303u) << 4);
    // this lane's 8 weights l = 8c..8c+7 of the quarter: scale 8h + 2j + c/2,
    // in scale dword 2h + j/2 (the same for every lane: no per-lane branch)
    // at byte (2j + c/2) % 4
    const int wq = 2 * h + (j >> 1);
    const uint32_t lo = wq == 0 ? r.s.x : wq == 1 ? r.s.y : wq == 2 ? r.s.z : r.s.w;
    const uint32_t hi = wq == 0 ? r.s.y : wq == 1 ? r.s.z : wq == 2 ? r.s.w : r.s4;
    const uint32_t sw = align_bytes(hi, lo, mis);
    const float sc = (float)(int)(int8_t)(sw >> (8 * ((2 * j + (c >> 1)) & 3)));
    const float off = -32.f * sc;
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        v[e] = __builtin_fmaf((float)((q0 >> (8 * e)) & 0xFFu), sc, off);  // sc * (q - 32), exact
        v[4 + e] = __builtin_fmaf((float)((q1 >> (8 * e)) & 0xFFu), sc, off);
    }
    split8(v, bh, bl);
}

// q8_0 and q4_0 (32-weight blocks): a step of 128 columns is blocks
// 4t .. 4t + 3, one MFMA chunk each; lane c holds the block's codes
// 8c .. 8c + 7 (q8_0: bytes 8c.. of the codes; q4_0: the low nibbles of
// bytes 8(c & 1).. for c < 2, their high nibbles for c >= 2).
template <> struct PwRaw<Q8_0> {
    uint32_t d[4];  // fp32 scales
    u32x2 q[4];     // codes 8c .. 8c + 7
};
template <> struct PwRaw<Q4_0> {
    uint32_t d[4];  // fp16 scales (low half)
    u32x2 q[4];     // nibble bytes 8(c & 1) .. +7, from the 4-byte boundary at or below them
    uint32_t t[2];  // blocks 0 and 2 of the step (2 bytes off that boundary): their last two bytes
};
template <> struct PwRaw<Q8_0_F16> {
    uint32_t d[4];  // fp16 scales (low half)
    u32x2 q[4];     // code bytes 8c .. 8c + 7, from the 4-byte boundary at or below them
    uint32_t t[2];  // blocks 0 and 2 of the step (codes 2 bytes off that boundary): codes 8c + 6, 8c + 7
};

// Byte offset of block b's codes for lane c, and q4_0's 4-byte window: rows
// start 4-byte aligned (row bytes are multiples of 144 when the columns are
// a multiple of 256), so an even block's nibble bytes sit 2 bytes past a
// 4-byte boundary and an odd block's on one.
__device__ __forceinline__ void pw_load_b32(PwRaw<Q8_0> &r, const uint8_t *wrow, int t, int c) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint8_t *blk = wrow + (int64_t)(4 * t + j) * 36;
        r.d[j] = ld_b32(blk);
        r.q[j] = ld_b64(blk + 4 + 8 * c);
    }
}
__device__ __forceinline__ void pw_load_b32(PwRaw<Q4_0> &r, const uint8_t *wrow, int t, int c) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint8_t *blk = wrow + (int64_t)(4 * t + j) * 18;
        const uint8_t *q = blk + 2 + 8 * (c & 1);
        r.d[j] = ld_b16(blk);
        if (j % 2 == 0) {
            // 2 bytes past a boundary: bytes q - 2 .. q + 5, then q + 6 .. q + 7
            // (a whole dword there would run past the block)
            r.q[j] = ld_b64(q - 2);
            r.t[j / 2] = ld_b16(q + 6);
        } else {
            r.q[j] = ld_b64(q);
        }
    }
}

// GGUF's Q8_0 (34-byte blocks): the same parity, fp16 d at the block's start
__device__ __forceinline__ void pw_load_b32(PwRaw<Q8_0_F16> &r, const uint8_t *wrow, int t, int c) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint8_t *blk = wrow + (int64_t)(4 * t + j) * 34;
        const uint8_t *q = blk + 2 + 8 * c;
        r.d[j] = ld_b16(blk);
        if (j % 2 == 0) {
            r.q[j] = ld_b64(q - 2);
            r.t[j / 2] = ld_b16(q + 6);
        } else {
            r.q[j] = ld_b64(q);
        }
    }
}

// B operand of chunk j: q8_0 codes as bf16 (integers of at most 8 bits: the
// top half of their fp32 pattern is exact); q4_0 codes as bf16 128 + n.
__device__ __forceinline__ u32x4 pw_codes(const PwRaw<Q8_0> &r, int j, int) {
    const u32x2 q = r.q[j];
    float f[8];
#pragma unroll
    for (int e = 0; e < 4; e++) {
        f[e] = (float)(int)(int8_t)(q.x >> (8 * e));
        f[4 + e] = (float)(int)(int8_t)(q.y >> (8 * e));
    }
    auto top2 = [](float lo, float hi) {
        return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, hi), __builtin_bit_cast(uint32_t, lo), 0x07060302u);
    };
    return u32x4{top2(f[0], f[1]), top2(f[2], f[3]), top2(f[4], f[5]), top2(f[6], f[7])};
}
__device__ __forceinline__ u32x4 pw_codes(const PwRaw<Q4_0> &r, int j, int c) {
    const u32x2 q = r.q[j];
    uint32_t w0 = q.x, w1 = q.y;
    if (j % 2 == 0) {  // realign: bytes q + 0 .. q + 7
        w0 = align_bytes(q.y, q.x, 2);
        w1 = align_bytes(r.t[j / 2], q.y, 2);
    }
    const int sh = 4 * (c >> 1);
    const uint32_t n0 = (w0 >> sh) & 0x0F0F0F0Fu, n1 = (w1 >> sh) & 0x0F0F0F0Fu;
    return u32x4{bf16_off_lo(n0), bf16_off_hi(n0), bf16_off_lo(n1), bf16_off_hi(n1)};
}
__device__ __forceinline__ u32x4 pw_codes(const PwRaw<Q8_0_F16> &r, int j, int) {
    u32x2 q = r.q[j];
    if (j % 2 == 0) q = u32x2{align_bytes(q.y, q.x, 2), align_bytes(r.t[j / 2], q.y, 2)};  // realign
    return codes_q8_0(q);
}
__device__ __forceinline__ float pw_scale(const PwRaw<Q8_0> &r, int j) { return __builtin_bit_cast(float, r.d[j]); }
__device__ __forceinline__ float pw_scale(const PwRaw<Q8_0_F16> &r, int j) {
    return half_bits_to_float(r.d[j] & 0xFFFFu);
}
__device__ __forceinline__ float pw_scale(const PwRaw<Q4_0> &r, int j) { return half_bits_to_float(r.d[j] & 0xFFFFu); }

// Q5_K, Q2_K, Q3_K (half h of a super-block) and Q5_1 (blocks 4t .. 4t + 3)
template <> struct PwRaw<Q5_K> : HRaw<Q5_K> {};
template <> struct PwRaw<Q2_K> : HRaw<Q2_K> {};
template <> struct PwRaw<Q3_K> : HRaw<Q3_K> {};
template <> struct PwRaw<Q5_1> : HRaw<Q5_1> {};
__device__ __forceinline__ void pw_load(HRaw<Q5_K> &r, const uint8_t *blk, int h, int c) {
    r.hd = ld_b128(blk);
#pragma unroll
    for (int i = 0; i < 2; i++) r.q[i] = ld_b64(blk + 48 + 32 * (2 * h + i) + 8 * c);
    r.qh = ld_b64(blk + 16 + 8 * c);
}
// (84-byte blocks keep the rows' 4-byte alignment)
__device__ __forceinline__ void pw_load(HRaw<Q2_K> &r, const uint8_t *blk, int h, int c) {
    r.q = ld_b64(blk + 16 + 32 * h + 8 * c);
    r.s = ld_b64(blk + 8 * h);
    r.dd = ld_b32(blk + 80);
}
// (the windows end at bytes 36, 100 and 108 of the aligned-down block, the
// tail is two 2-byte loads: nothing is read past the block)
__device__ __forceinline__ void pw_load(HRaw<Q3_K> &r, const uint8_t *blk, int h, int c) {
    r.mis = (uint32_t)(uintptr_t)blk & 3u;
    const uint8_t *A0 = blk - r.mis;
    r.hm = ld_b96(A0 + 8 * c);
    r.q = ld_b96(A0 + 32 + 32 * h + 8 * c);
    r.s = ld_b96(A0 + 96);
    r.tail = ld_b16(blk + 106) | (ld_b16(blk + 108) << 16);
}
__device__ __forceinline__ void pw_load_b32(HRaw<Q5_1> &r, const uint8_t *wrow, int t, int c) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
        const uint8_t *blk = wrow + (int64_t)(4 * t + j) * 24;
        r.dq[j] = ld_b64(blk);
        r.q[j] = ld_b64(blk + 8 + 8 * (c & 1));
    }
}
template <int F>
__device__ __forceinline__ void pw_dec(const HRaw<F> &r, int h, int j, int c, u32x4 &bh, u32x4 &bl) {
    h_operands<F>(r, h, j, c, bh, bl);
}

// Load instructions a step issues for its weights (at least: the compiler
// may merge adjacent loads). After a step's X tile loads come its weight
// loads; waiting until no more than this many loads are outstanding
// therefore covers the tile (the load counter counts in order), and leaves
// (at least) the last weight loads in flight.
template <int F> struct PwWLoads;
template <> struct PwWLoads<Q4_K> { static constexpr int N = 3; };  // 16 + 8 + 8 bytes
template <> struct PwWLoads<Q6_K> { static constexpr int N = 4; };  // 3 x 12 + 16 + (2 + 2) bytes
template <> struct PwWLoads<Q8_0> { static constexpr int N = 4; };  // 4 x (4 + 8) bytes
template <> struct PwWLoads<Q4_0> { static constexpr int N = 6; };  // 4 x 2 + 4 x 8 + 2 x 2 bytes
// (a block's loads may merge into one; four blocks take at least four)
template <> struct PwWLoads<Q8_0_F16> { static constexpr int N = 4; };  // 4 x 2 + 4 x 8 + 2 x 2 bytes
template <> struct PwWLoads<Q5_K> { static constexpr int N = 4; };       // 16 + 3 x 8 bytes
template <> struct PwWLoads<Q2_K> { static constexpr int N = 3; };       // 8 + 8 + 4 bytes
template <> struct PwWLoads<Q3_K> { static constexpr int N = 4; };       // 3 x 12 + (2 + 2) bytes
template <> struct PwWLoads<Q5_1> { static constexpr int N = 4; };       // 4 x (8 + 8) bytes (at least 4)

// Workgroups per CU the register budget is sized for (measured at M = 64
// and 512 on the 5632 x 2048, 2048 x 5632 and 4096 x 11008 shapes); two
// 128-token tiles fill 128 KiB of LDS.
template <int F, int TOK> constexpr int pw_occupancy() {
    return TOK == 128 ? 2 : F == Q4_K ? 4 : F == Q6_K ? 2 : 3;
}

typedef __attribute__((address_space(3))) void lds_void;

template <int F, int KH, int TOK>
__global__ __launch_bounds__(256, (pw_occupancy<F, TOK>())) void gemm_pw_kernel(const uint8_t *W, int rows, int nb,
                                                                                int64_t row_bytes, const uint16_t *X,
                                                                                int M, float *Y) {
    // (no __restrict__ on W and X: it would let the compiler move weight
    // loads across the fences that keep each step's loads in order)
    static_assert(TOK == 64 || TOK == 128, "tokens per workgroup");
    constexpr int BYTES = Layout<F>::BYTES;
    constexpr int MT = TOK / 16;    // M tiles per wave
    constexpr int NJ = TOK / 16;    // X tile loads per thread and step (TOK * 16 chunks / 256 threads)
    constexpr int TILE = TOK * 128; // bf16 per X tile
    // two buffers as two objects: a read of one is then known not to touch
    // the other one's loads in flight
    __shared__ __attribute__((aligned(16))) uint16_t xs0[TILE];
    __shared__ __attribute__((aligned(16))) uint16_t xs1[TILE];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, c = lane >> 4;
    const int m0 = (int)blockIdx.y * TOK;
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
    const int tl = t0 + nsteps - 1;

    // X tile load i of wave w fills chunk slots 256 i + 64 w + lane (the
    // direct loads put lane l's 16 bytes at 16 l past the instruction's LDS
    // address): token 16 i + 4 w + lane / 16, slot lane % 16, which holds
    // column chunk (lane % 16) ^ (token % 16); tokens past M load token
    // M - 1 (their products are not stored)
    const int r0 = 4 * wave + (lane >> 4);
    const int kc = (lane & 15) ^ (r0 & 15);
    const uint16_t *xrow[NJ];
#pragma unroll
    for (int i = 0; i < NJ; i++) xrow[i] = X + (int64_t)min(m0 + 16 * i + r0, M - 1) * ldx + 8 * kc;
    auto x_load = [&](int t, uint16_t *dst) {
#pragma unroll
        for (int i = 0; i < NJ; i++)
            __builtin_amdgcn_global_load_lds(static_cast<const void *>(xrow[i] + (int64_t)t * 128),
                                             (lds_void *)(dst + 2048 * i + 512 * wave), 16, 0, 0);
    };
    auto w_load = [&](PwRaw<F> &r, int t) {
        if constexpr (Layout<F>::QK == 256)
            pw_load(r, wrow + (int64_t)(t >> 1) * BYTES, t & 1, c);
        else
            pw_load_b32(r, wrow, t, c);
    };
    // lane (n, c) reads the A operand of M tile a, chunk j (token 16 a + n,
    // column chunk 4 j + c) at so[j] + 2048 a
    int so[4];
#pragma unroll
    for (int j = 0; j < 4; j++) so[j] = n * 128 + (((4 * j + c) ^ n) << 3);

    f32x4 acc[MT], sbacc[F == Q6_K ? MT : 1];
#pragma unroll
    for (int a = 0; a < MT; a++) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    PwRaw<F> wb[3];
    x_load(t0, xs0);
    w_load(wb[0], t0);
    w_load(wb[1], min(t0 + 1, tl));
    __builtin_amdgcn_s_waitcnt(0);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // one step: the 4 chunks of half t, the X tile in xb
    auto compute = [&](const PwRaw<F> &r, int t, const uint16_t *xb) {
        // (the half stays opaque to the compiler: known per unrolled step,
        // it would make parts of the 16-byte loads dead, and their registers
        // would be reused while the loads are in flight)
        int h = t & 1;
        asm volatile("" : "+s"(h));
        if constexpr (F == Q8_0 || F == Q4_0 || F == Q8_0_F16) {
            // one product per block and M tile, scaled by the block's d
            // (q4_0: the offset product, X against -136 = -(128 + 8), is the
            // code product's accumulator)
            const u32x4 m136 = u32x4{0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u};
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const u32x4 bw = pw_codes(r, j, c);
                const float d = pw_scale(r, j);
                bf16x8 av[MT];
                f32x4 P[MT];
#pragma unroll
                for (int a = 0; a < MT; a++) av[a] = *reinterpret_cast<const bf16x8 *>(xb + 2048 * a + so[j]);
#pragma unroll
                for (int a = 0; a < MT; a++)
                    P[a] = F == Q4_0 ? __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                           av[a], __builtin_bit_cast(bf16x8, m136), f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0)
                                     : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int a = 0; a < MT; a++)
                    P[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bw), P[a], 0, 0, 0);
#pragma unroll
                for (int a = 0; a < MT; a++) acc[a] += d * P[a];
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; j++) {
                u32x4 bh, bl;
                if constexpr (F == Q4_K)
                    pw_dec(r, h, j, bh, bl);
                else
                    pw_dec(r, h, j, c, bh, bl);
                bf16x8 av[MT];
#pragma unroll
                for (int a = 0; a < MT; a++) av[a] = *reinterpret_cast<const bf16x8 *>(xb + 2048 * a + so[j]);
                if constexpr (F != Q6_K) {
#pragma unroll
                    for (int a = 0; a < MT; a++)
                        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bh), acc[a],
                                                                        0, 0, 0);
#pragma unroll
                    for (int a = 0; a < MT; a++)
                        acc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bl), acc[a],
                                                                        0, 0, 0);
                } else {
                    // the super-block's sums start at its first chunk
                    const bool first = h == 0 && j == 0;
#pragma unroll
                    for (int a = 0; a < MT; a++)
                        sbacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            av[a], __builtin_bit_cast(bf16x8, bh), first ? f32x4{0.f, 0.f, 0.f, 0.f} : sbacc[a], 0, 0,
                            0);
#pragma unroll
                    for (int a = 0; a < MT; a++)
                        sbacc[a] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], __builtin_bit_cast(bf16x8, bl),
                                                                          sbacc[a], 0, 0, 0);
                }
            }
            if constexpr (F == Q6_K) {
                if (h == 1) {  // the super-block is complete: its d scales its sums
                    const float d = half_bits_to_float(r.s4 >> 16);
#pragma unroll
                    for (int a = 0; a < MT; a++) acc[a] += d * sbacc[a];
                }
            }
        }
    };
    // Step k of a round of 6 (buffer and slot indices are compile-time): the
    // X tile of step t + 1 into the other LDS buffer (read last in step t - 1,
    // before the barrier that ended it), the weights of step t + 2, the
    // multiply of step t; then wait for this wave's tile loads (not the
    // weight loads after them) and meet the other waves, after which the
    // whole tile of step t + 1 is in LDS. The loads are unconditional (past
    // the last step they reload it). The empty asm statements keep the
    // compiler from moving loads across these groups; the barrier is the
    // bare instruction, without the fence of __syncthreads, which would wait
    // for every load.
    constexpr int NW = PwWLoads<F>::N;
    constexpr int WAIT_X = (NW & 15) | (7 << 4) | (0 << 8) | ((NW >> 4) << 14);  // vmcnt(NW) lgkmcnt(0)
#define QK_PW_FENCE()                \
    asm volatile("" ::: "memory");   \
    __builtin_amdgcn_sched_barrier(0)
#define QK_PW_STEP(K)                                          \
    {                                                          \
        const int t = t0 + i + (K);                            \
        x_load(min(t + 1, tl), ((K) + 1) % 2 ? xs1 : xs0);     \
        QK_PW_FENCE();                                         \
        w_load(wb[((K) + 2) % 3], min(t + 2, tl));             \
        QK_PW_FENCE();                                         \
        compute(wb[(K) % 3], t, (K) % 2 ? xs1 : xs0);          \
        QK_PW_FENCE();                                         \
        __builtin_amdgcn_s_waitcnt(WAIT_X);                    \
        __builtin_amdgcn_s_barrier();                          \
        QK_PW_FENCE();                                         \
        if (i + (K) + 1 >= nsteps) break;                      \
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
#undef QK_PW_FENCE
    // (the last steps' reloads land before the workgroup ends)
    __builtin_amdgcn_s_waitcnt(0);

    // lane holds tokens 16a + 4c + i of row rbase + n
    const int r = rbase + n;
#pragma unroll
    for (int a = 0; a < MT; a++)
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

// Tokens per prefill workgroup (QK_TUNE_PREFILL_TOKENS sets it): 128 for
// q8_0, q4_0 and GGUF's Q8_0 from M = 128, and for the others from M = 192
// where the 128-token tiles number more than half the CUs, or exactly half
// on rows of 16 or more super-blocks (each decoded weight then feeds 8 M
// tiles); else 64. Measured over M = 128 .. 1024 on Q4_K 5632 x 2048 and
// 11008 x 4096, Q6_K 2048 x 5632 and 4096 x 11008, q8_0 and q4_0 5632 x
// 2048, with the split rule below: within 3.2 % of the fastest of the four
// tile / split choices in every case (M = 512: Q4_K 5632 x 2048 34.6 us,
// Q6_K 2048 x 5632 43.9, q8_0 44.2 against 57.3 with 64-token tiles); and
// over M = 32 .. 512 on twelve shapes of 1024 .. 8192 rows: at exactly half
// the CUs short rows ran faster with 64-token tiles (2048 x 2048 at M = 512:
// Q4_K 20.5 against 24.0 us, Q6_K 22.4 against 25.0), while 4096 x 11008
// Q6_K at M = 256 kept 128 (76.8 against 78.5).
template <int F> inline int pw_tokens(int64_t rows, int64_t cols, int64_t M) {
    const int f = tuning(QK_TUNE_PREFILL_TOKENS);
    if (f == 64 || f == 128) return f;
    if constexpr (F == Q8_0 || F == Q4_0 || F == Q8_0_F16) return M >= 128 ? 128 : 64;
    const int64_t t128 = ((rows + 63) / 64) * ((M + 127) / 128), half = device_cu_count() / 2;
    return M >= 192 && (t128 > half || (t128 == half && cols / 256 >= 16)) ? 128 : 64;
}

// K split over two workgroups (QK_TUNE_GEMM_KSPLIT = 1/2 forces it): where
// the tiles number at most half the CUs, or where the rows are long (16 or
// more super-blocks) and the tiles number at most the CUs (twice the CUs
// with 64-token tiles). On rows of 8 super-blocks the zeroing launch and
// the atomic adds cost more than the idle CUs from 176 tiles up (q8_0 5632
// x 2048 at M = 256: 26.6 us unsplit, 33.3 split); on long rows the split
// pays up to 512 tiles (Q4_K 11008 x 4096 at M = 128: 39.8 against 46.2).
inline bool pw_split(int64_t tiles, int64_t nb, int tok) {
    const int64_t cus = device_cu_count();
    return tiles <= cus / 2 || (nb >= 16 && tiles <= cus * (tok == 64 ? 2 : 1));
}

template <int F, int KH, int TOK>
static hipError_t launch_pw(const uint8_t *W, int64_t rows, int64_t cols, int64_t row_bytes, const uint16_t *X,
                            int64_t M, float *Y, hipStream_t stream) {
    if (KH > 1) {
        // each half needs a step: with one 256-column step the first half
        // would have none and its prologue would read before W and X
        if (cols / 256 < 2) return hipErrorInvalidValue;
        const hipError_t ez = launch_fill_zero(Y, M * rows, stream);
        if (ez != hipSuccess) return ez;
    }
    const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((M + TOK - 1) / TOK), (unsigned)KH);
    hipLaunchKernelGGL((gemm_pw_kernel<F, KH, TOK>), grid, dim3(256), 0, stream, W, (int)rows, (int)(cols / 256),
                       row_bytes, X, (int)M, Y);
    return hipGetLastError();
}

// Which kernel a GEMM of this format, shape and M runs (a qk_gemm_path):
// for rows of whole 256-column steps the few-token kernel for M <= 16 and
// the prefill kernel above, else the row kernel. QK_TUNE_GEMM_PATH forces
// one where it applies (the few-token kernel takes at most 16 rows of X).
// (Below 2^26 columns the few-token kernel's raw buffers, 8 rows of W and
// 16 rows of X, stay under 2 GiB.)
template <int F> static int gemm_path_t(int64_t rows, int64_t cols, int64_t M) {
    // (the K-quants' rows are always whole steps; the 32-weight block
    // formats' rows when their block count is a multiple of 8)
    if (rows < (int64_t(1) << 30) && M < (int64_t(1) << 30) && cols < (int64_t(1) << 26) && cols % 256 == 0) {
        const int force = tuning(QK_TUNE_GEMM_PATH);
        if (force == QK_GEMM_PATH_ROWS) return QK_GEMM_PATH_ROWS;
        if (force == QK_GEMM_PATH_PREFILL) return QK_GEMM_PATH_PREFILL;
        if (force == QK_GEMM_PATH_FEW && M <= 16) return QK_GEMM_PATH_FEW;
        return M <= 16 ? QK_GEMM_PATH_FEW : QK_GEMM_PATH_PREFILL;
    }
    return QK_GEMM_PATH_ROWS;
}

template <int F>
static hipError_t launch_gemm_t(const uint8_t *W, int64_t rows, int64_t cols, const uint16_t *X, int64_t M, float *Y,
                                hipStream_t stream) {
    constexpr int QK = Layout<F>::QK, BYTES = Layout<F>::BYTES;
    const int64_t row_bytes = cols / QK * BYTES;
    const int path = gemm_path_t<F>(rows, cols, M);
    if (path == QK_GEMM_PATH_PREFILL) {
        const int ksf = tuning(QK_TUNE_GEMM_KSPLIT);
        const int tok = pw_tokens<F>(rows, cols, M);
        const int64_t tiles = ((rows + 63) / 64) * ((M + tok - 1) / tok);
        // (the split halves whole 256-column steps: it needs two)
        const bool split = cols / 256 >= 2 && (ksf == 2 || (ksf < 0 && pw_split(tiles, cols / 256, tok)));
        if (tok == 128)
            return split ? launch_pw<F, 2, 128>(W, rows, cols, row_bytes, X, M, Y, stream)
                         : launch_pw<F, 1, 128>(W, rows, cols, row_bytes, X, M, Y, stream);
        return split ? launch_pw<F, 2, 64>(W, rows, cols, row_bytes, X, M, Y, stream)
                     : launch_pw<F, 1, 64>(W, rows, cols, row_bytes, X, M, Y, stream);
    }
    if (path == QK_GEMM_PATH_FEW) return launch_few<F>(W, rows, cols, row_bytes, X, M, Y, stream);
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
    case Q8_0: return gemm_path_t<Q8_0>(rows, cols, M);
    case Q4_0: return gemm_path_t<Q4_0>(rows, cols, M);
    case Q8_0_F16: return gemm_path_t<Q8_0_F16>(rows, cols, M);
    case Q5_1: return gemm_path_t<Q5_1>(rows, cols, M);
    case Q5_K: return gemm_path_t<Q5_K>(rows, cols, M);
    case Q2_K: return gemm_path_t<Q2_K>(rows, cols, M);
    case Q3_K: return gemm_path_t<Q3_K>(rows, cols, M);
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
