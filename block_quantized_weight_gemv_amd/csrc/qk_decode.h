// qk_decode.h — bit-exact decode of four consecutive weights of one block.
//
// Used by the dequantisation kernel and by the generic (any-alignment) GEMV
// path. Each weight is evaluated in fp32 in the pages' order with explicit
// round-to-nearest operations, so no contraction can change its bits:
//   Q4_K  (d*scale)*q - dmin*min   ("picoLM, in Python", §2 K-quants)
//   Q6_K  (d*scale)*q              ("PicoLM Q6_K量化Bug调试全记录", 原理)
//   Q8_0  scale*q,  Q4_0  d*(nibble-8)   (PETIT README, "How the pieces match")
//   Q8_0_F16  d*q;  Q5_1  q*d + m;  Q5_K  (d*scale)*q - dmin*min;
//   Q2_K  (d*scale)*q - dmin*min;  Q3_K  (d*scale)*q   (the ggml formats)
// Only 2-byte loads are used for Q6_K, Q4_0, Q8_0_F16 and Q3_K, whose blocks
// (210, 18, 34 and 110 bytes) are only 2-byte aligned in general.
#pragma once

#include "qk_formats.h"

namespace qk {

// Q4_K scale and min of sub-block j from the 12 packed bytes, given as three
// little-endian dwords (packed bytes 0..3, 4..7, 8..11).
__device__ __forceinline__ void q4k_scale_min(uint32_t p0, uint32_t p1, uint32_t p2, int j,
                                              uint32_t &sc, uint32_t &mn) {
    if (j < 4) {
        sc = (p0 >> (8 * j)) & 63u;
        mn = (p1 >> (8 * j)) & 63u;
    } else {
        const int i = j - 4;
        sc = ((p2 >> (8 * i)) & 0xFu) | (((p0 >> (8 * i + 6)) & 3u) << 4);
        mn = ((p2 >> (8 * i + 4)) & 0xFu) | (((p1 >> (8 * i + 6)) & 3u) << 4);
    }
}

__device__ __forceinline__ uint32_t ld_u32_via_u16(const uint8_t *p) {
    return ld_b16(p) | (ld_b16(p + 2) << 16);
}

// out[0..3] = weights i0..i0+3 of the block at blk (i0 a multiple of 4).
template <int F>
__device__ __forceinline__ void decode4(const uint8_t *blk, int i0, float out[4]);

template <>
__device__ __forceinline__ void decode4<Q4_K>(const uint8_t *blk, int i0, float out[4]) {
    // Q4_K blocks start 16-byte aligned (base 16-byte aligned, 144 = 9*16).
    const uint32_t h0 = ld_b32(blk), p0 = ld_b32(blk + 4), p1 = ld_b32(blk + 8), p2 = ld_b32(blk + 12);
    const int g = i0 / 64, r = i0 % 64, hi = r >= 32, l = r % 32;
    const uint32_t qd = ld_b32(blk + 16 + 32 * g + l);
    uint32_t sc, mn;
    q4k_scale_min(p0, p1, p2, 2 * g + hi, sc, mn);
    const float d = half_bits_to_float(h0 & 0xFFFFu);
    const float dmin = half_bits_to_float(h0 >> 16);
    const float dsc = __fmul_rn(d, (float)sc);
    const float m = __fmul_rn(dmin, (float)mn);
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t q = (qd >> (8 * k + 4 * hi)) & 0xFu;
        out[k] = __fsub_rn(__fmul_rn(dsc, (float)q), m);
    }
}

template <>
__device__ __forceinline__ void decode4<Q6_K>(const uint8_t *blk, int i0, float out[4]) {
    const int h = i0 / 128, k = (i0 % 128) / 32, l = i0 % 32;
    const uint32_t ql = ld_u32_via_u16(blk + 64 * h + 32 * (k & 1) + l);
    const uint32_t qh = ld_u32_via_u16(blk + 128 + 32 * h + l);
    const int si = 8 * h + 2 * k + l / 16;  // one scale per 16 weights
    const uint32_t spair = ld_b16(blk + 192 + (si & ~1));
    const int sc = (int)(int8_t)(spair >> (8 * (si & 1)));
    const float d = half_bits_to_float(ld_b16(blk + 208));
    const float dsc = __fmul_rn(d, (float)sc);
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const uint32_t lo = (ql >> (8 * c + (k >= 2 ? 4 : 0))) & 0xFu;
        const uint32_t hi2 = (qh >> (8 * c + 2 * k)) & 3u;
        const int q = (int)(lo | (hi2 << 4)) - 32;
        out[c] = __fmul_rn(dsc, (float)q);
    }
}

template <>
__device__ __forceinline__ void decode4<Q8_0>(const uint8_t *blk, int i0, float out[4]) {
    // 36-byte blocks keep 4-byte alignment.
    const float s = __builtin_bit_cast(float, ld_b32(blk));
    const uint32_t q = ld_b32(blk + 4 + i0);
#pragma unroll
    for (int c = 0; c < 4; c++) out[c] = __fmul_rn(s, (float)(int)(int8_t)(q >> (8 * c)));
}

template <>
__device__ __forceinline__ void decode4<Q4_0>(const uint8_t *blk, int i0, float out[4]) {
    const float d = half_bits_to_float(ld_b16(blk));
    const int hi = i0 >= 16;
    const uint32_t q = ld_u32_via_u16(blk + 2 + (i0 % 16));
#pragma unroll
    for (int c = 0; c < 4; c++) out[c] = __fmul_rn(d, (float)((int)((q >> (8 * c + 4 * hi)) & 0xFu) - 8));
}

template <>
__device__ __forceinline__ void decode4<Q8_0_F16>(const uint8_t *blk, int i0, float out[4]) {
    const float d = half_bits_to_float(ld_b16(blk));
    const uint32_t q = ld_u32_via_u16(blk + 2 + i0);
#pragma unroll
    for (int c = 0; c < 4; c++) out[c] = __fmul_rn(d, (float)(int)(int8_t)(q >> (8 * c)));
}

template <>
__device__ __forceinline__ void decode4<Q5_1>(const uint8_t *blk, int i0, float out[4]) {
    // 24-byte blocks keep 8-byte alignment.
    const uint32_t dm = ld_b32(blk), qh = ld_b32(blk + 4);
    const float d = half_bits_to_float(dm & 0xFFFFu), m = half_bits_to_float(dm >> 16);
    const int hi = i0 >= 16;
    const uint32_t q = ld_b32(blk + 8 + (i0 % 16));
#pragma unroll
    for (int c = 0; c < 4; c++) {
        // weight i0+c: its nibble, and bit i0+c of qh as the fifth bit
        const uint32_t v = ((q >> (8 * c + 4 * hi)) & 0xFu) | (((qh >> (i0 + c)) & 1u) << 4);
        out[c] = __fadd_rn(__fmul_rn((float)v, d), m);
    }
}

template <>
__device__ __forceinline__ void decode4<Q5_K>(const uint8_t *blk, int i0, float out[4]) {
    const uint32_t h0 = ld_b32(blk), p0 = ld_b32(blk + 4), p1 = ld_b32(blk + 8), p2 = ld_b32(blk + 12);
    const int g = i0 / 64, r = i0 % 64, hi = r >= 32, l = r % 32, j = 2 * g + hi;
    const uint32_t qd = ld_b32(blk + 48 + 32 * g + l);
    const uint32_t qh = ld_b32(blk + 16 + l);
    uint32_t sc, mn;
    q4k_scale_min(p0, p1, p2, j, sc, mn);
    const float d = half_bits_to_float(h0 & 0xFFFFu);
    const float dmin = half_bits_to_float(h0 >> 16);
    const float dsc = __fmul_rn(d, (float)sc);
    const float m = __fmul_rn(dmin, (float)mn);
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t q = ((qd >> (8 * k + 4 * hi)) & 0xFu) | (((qh >> (8 * k + j)) & 1u) << 4);
        out[k] = __fsub_rn(__fmul_rn(dsc, (float)q), m);
    }
}

template <>
__device__ __forceinline__ void decode4<Q2_K>(const uint8_t *blk, int i0, float out[4]) {
    // 84-byte blocks keep 4-byte alignment.
    const int h = i0 / 128, j = (i0 % 128) / 32, l = i0 % 32, s = i0 / 16;
    const uint32_t qd = ld_b32(blk + 16 + 32 * h + l);
    const uint32_t sb = (ld_b32(blk + (s & ~3)) >> (8 * (s & 3))) & 0xFFu;
    const uint32_t dd = ld_b32(blk + 80);
    const float dl = __fmul_rn(half_bits_to_float(dd & 0xFFFFu), (float)(sb & 0xFu));
    const float ml = __fmul_rn(half_bits_to_float(dd >> 16), (float)(sb >> 4));
#pragma unroll
    for (int c = 0; c < 4; c++) out[c] = __fsub_rn(__fmul_rn(dl, (float)((qd >> (8 * c + 2 * j)) & 3u)), ml);
}

__device__ __forceinline__ uint32_t byte_via_u16(const uint8_t *base, int k) {
    return (ld_b16(base + (k & ~1)) >> (8 * (k & 1))) & 0xFFu;
}

template <>
__device__ __forceinline__ void decode4<Q3_K>(const uint8_t *blk, int i0, float out[4]) {
    const int h = i0 / 128, j = (i0 % 128) / 32, l = i0 % 32, s = i0 / 16;
    const uint32_t qd = ld_u32_via_u16(blk + 32 + 32 * h + l);
    const uint32_t hm = ld_u32_via_u16(blk + l);
    const uint32_t lo4 = s < 8 ? (byte_via_u16(blk + 96, s) & 0xFu) : (byte_via_u16(blk + 96, s - 8) >> 4);
    const uint32_t hi2 = (byte_via_u16(blk + 96, 8 + s % 4) >> (2 * (s / 4))) & 3u;
    const int sc = (int)(lo4 | (hi2 << 4)) - 32;
    const float dsc = __fmul_rn(half_bits_to_float(ld_b16(blk + 108)), (float)sc);
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const int q2 = (int)((qd >> (8 * c + 2 * j)) & 3u);
        const int q = q2 - (((hm >> (8 * c + 4 * h + j)) & 1u) ? 0 : 4);
        out[c] = __fmul_rn(dsc, (float)q);
    }
}

}  // namespace qk
