// qk_formats.h — block layouts and device-side field readers for the four
// formats, GPU side.
//
// Layouts (byte offsets inside one block):
//   Q4_K (144 B / 256 weights) — "picoLM, in Python", "§2 — K-quants":
//       0 d (fp16) | 2 dmin (fp16) | 4..15 packed 6-bit scales/mins | 16..143 nibbles
//       Nibble byte 32g+l: low nibble = weight 64g+l (sub-block 2g), high
//       nibble = weight 64g+32+l (sub-block 2g+1). Sub-blocks 0..3 keep scale
//       and min in the low 6 bits of packed bytes j and j+4; sub-blocks 4..7
//       take their low 4 bits from packed byte j+4 (scale: low nibble, min:
//       high nibble) and their top 2 bits from the top 2 bits of packed byte
//       j-4 (scale) or j (min).
//   Q6_K (210 B / 256 weights) — "PicoLM Q6_K量化Bug调试全记录", 原理:
//       0..127 ql (low 4 bits) | 128..191 qh (high 2 bits) | 192..207 int8
//       scales[16] | 208 d (fp16). Weight 128h+32k+l (half h, quarter k,
//       l < 32): low 4 bits from ql[64h+32(k&1)+l] (low nibble if k < 2, else
//       high nibble), high 2 bits = bits 2k..2k+1 of qh[32h+l], code - 32;
//       scale = scales[8h + 2k + l/16] (one scale per 16 weights).
//   Q8_0 (36 B / 32) and Q4_0 (18 B / 32) — PETIT README, "How the pieces
//       match": fp32 scale + 32 int8; fp16 scale + 16 nibble bytes with byte
//       j = weight j (low nibble) | weight j+16 (high nibble), nibble - 8.
//   The ggml-specification formats the K-quants page names (it gives only
//   Q2_K's size, 84 bytes per 256 weights, and takes ggml as the formats'
//   source of truth — "picoLM, in Python", §2, "Verify against the spec";
//   "Exercises" names Q5_K and Q5_1):
//   Q8_0_F16 (34 B / 32): 0 d (fp16) | 2 int8 q[32]; d*q (GGUF's Q8_0).
//   Q5_1 (24 B / 32): 0 d | 2 m (fp16) | 4 qh (uint32) | 8 nibbles[16];
//       byte j: weight j = low nibble + 16*bit j of qh, weight j+16 = high
//       nibble + 16*bit j+16; q*d + m.
//   Q5_K (176 B / 256): Q4_K's 16-byte header | 16 qh[32] | 48 nibbles[128];
//       weight 64g+l (low nibble of byte 32g+l) adds 16*bit 2g of qh[l],
//       weight 64g+32+l (high nibble) 16*bit 2g+1; as Q4_K otherwise.
//   Q2_K (84 B / 256): 0 scales[16] (low nibble scale, high nibble min, one
//       per 16 weights) | 16 qs[64] | 80 d | 82 dmin; weight 128h+32j+l =
//       bits 2j..2j+1 of qs[32h+l]; d*scale*q - dmin*min.
//   Q3_K (110 B / 256): 0 hmask[32] | 32 qs[64] | 96 packed 6-bit scales[12]
//       | 108 d; weight 128h+32j+l = (bits 2j..2j+1 of qs[32h+l]) - 4 unless
//       bit 4h+j of hmask[l] is set; scale s (per 16 weights): low 4 bits in
//       byte s (s < 8) or the high nibble of byte s-8, top 2 bits at bit
//       2(s/4) of byte 8 + s%4, stored +32; d*scale*q.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qk {

enum Format : int { Q4_0 = 1, Q8_0 = 2, Q4_K = 3, Q6_K = 4, Q8_0_F16 = 5, Q5_1 = 6, Q5_K = 7, Q2_K = 8, Q3_K = 9 };

template <int F> struct Layout;
template <> struct Layout<Q4_K> { static constexpr int QK = 256, BYTES = 144; };
template <> struct Layout<Q6_K> { static constexpr int QK = 256, BYTES = 210; };
template <> struct Layout<Q8_0> { static constexpr int QK = 32, BYTES = 36; };
template <> struct Layout<Q4_0> { static constexpr int QK = 32, BYTES = 18; };
template <> struct Layout<Q8_0_F16> { static constexpr int QK = 32, BYTES = 34; };
template <> struct Layout<Q5_1> { static constexpr int QK = 32, BYTES = 24; };
template <> struct Layout<Q5_K> { static constexpr int QK = 256, BYTES = 176; };
template <> struct Layout<Q2_K> { static constexpr int QK = 256, BYTES = 84; };
template <> struct Layout<Q3_K> { static constexpr int QK = 256, BYTES = 110; };

// Bits per weight printed on the pages: Q4_K 4.50, Q6_K 6.56, q4_0 4.5.
static_assert(Layout<Q4_K>::BYTES == 2 + 2 + 12 + 128, "Q4_K block size");
static_assert(Layout<Q6_K>::BYTES == 128 + 64 + 16 + 2, "Q6_K block size");
static_assert(Layout<Q8_0>::BYTES == 4 + 32, "q8_0 block size");
static_assert(Layout<Q4_0>::BYTES == 2 + 16, "q4_0 block size");
static_assert(Layout<Q4_K>::BYTES * 8 * 100 / Layout<Q4_K>::QK == 450, "Q4_K is 4.50 bits/weight");
static_assert(Layout<Q6_K>::BYTES * 8 * 1000 / Layout<Q6_K>::QK == 6562, "Q6_K is 6.56 bits/weight");
static_assert(Layout<Q4_0>::BYTES * 8 * 10 / Layout<Q4_0>::QK == 45, "q4_0 is 4.5 bits/weight");
static_assert(Layout<Q2_K>::BYTES == 16 + 64 + 2 + 2, "Q2_K block size");
static_assert(Layout<Q2_K>::BYTES * 8 * 100 / Layout<Q2_K>::QK == 262, "Q2_K is 2.62 bits/weight");
static_assert(Layout<Q3_K>::BYTES == 32 + 64 + 12 + 2, "Q3_K block size");
static_assert(Layout<Q5_K>::BYTES == 2 + 2 + 12 + 32 + 128, "Q5_K block size");
static_assert(Layout<Q5_1>::BYTES == 2 + 2 + 4 + 16, "Q5_1 block size");
static_assert(Layout<Q8_0_F16>::BYTES == 2 + 32, "fp16-scale Q8_0 block size");

// Q4_K blocks are 9 x 16 bytes, so with a 16-byte aligned base every block
// and every 16-byte piece of one is 16-byte aligned.
static_assert(Layout<Q4_K>::BYTES % 16 == 0, "Q4_K blocks keep 16-byte alignment");
static_assert(Layout<Q5_K>::BYTES % 16 == 0, "Q5_K blocks keep 16-byte alignment");
static_assert(Layout<Q5_1>::BYTES % 8 == 0 && Layout<Q2_K>::BYTES % 4 == 0, "Q5_1 / Q2_K blocks keep 4-byte alignment");

// ---------------------------------------------------------------- loads

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes from a 4-byte aligned address (one global_load_dwordx4).
__device__ __forceinline__ u32x4 ld_b128(const uint8_t *p) {
    u32x4 v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 16);
    return v;
}

// Streaming variants (cache policy "nt"): for bytes read exactly once.
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
__device__ __forceinline__ u32x4 ld_b128_nt(const uint8_t *p) {
    const u32x4_a4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_a4 *>(__builtin_assume_aligned(p, 4)));
    return u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ uint32_t ld_b32_nt(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(__builtin_assume_aligned(p, 4)));
}

// 8 bytes from a 4-byte aligned address (one global_load_dwordx2).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 ld_b64(const uint8_t *p) {
    u32x2 v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 8);
    return v;
}

__device__ __forceinline__ uint32_t ld_b32(const uint8_t *p) {
    uint32_t v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 4), 4);
    return v;
}

__device__ __forceinline__ uint32_t ld_b16(const uint8_t *p) {
    uint16_t v;
    __builtin_memcpy(&v, __builtin_assume_aligned(p, 2), 2);
    return v;
}

// The last four bytes of a Q6_K block as one dword: scales 14 and 15 in the
// low half, d in the high half (bytes 206..209). Read as two 2-byte loads,
// so that no read leaves the block: a dword window at the 4-byte boundary
// at or below byte 206 would end 2 bytes past a block that starts 4-byte
// aligned, past the matrix if that block is its last.
__device__ __forceinline__ uint32_t q6k_tail(const uint8_t *blk) { return ld_b16(blk + 206) | (ld_b16(blk + 208) << 16); }

// binary16 bits -> fp32 (exact; v_cvt_f32_f16).
__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// bytes {hi:lo} >> 8*shift, low 32 bits (v_alignbyte_b32); shift in 0..3.
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t shift) {
    return __builtin_amdgcn_alignbyte(hi, lo, shift);
}

}  // namespace qk
