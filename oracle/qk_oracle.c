/*
 * qk_oracle.c — plain, slow CPU oracle for block-quantized weight decoding
 * and for the GEMV / GEMM built on it.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the package smoke check and the
 * benchmark's CPU-baseline leg load this file's library. The GPU library
 * never includes, links or calls it, and it shares no code, header, table or
 * constant with the GPU path: every layout below is written out again here,
 * straight from the pages that define it.
 *
 * Sources (page, section):
 *   [S21]   "picoLM, in Python" (llminference.xinbetween.com/en/s21/),
 *           "§2 — K-quants": the Q4_K super-block (256 weights in 144 bytes:
 *           fp16 d, fp16 dmin, eight 6-bit scales and eight 6-bit mins packed
 *           into 12 bytes, 128 bytes of nibbles) and its dequantiser.
 *   [Q6K]   "PicoLM Q6_K量化Bug调试全记录" (cf-1.com/news/5431322/),
 *           section "原理" (principle): the Q6_K block holds ql[128] (low 4
 *           bits), qh[64] (high 2 bits), int8 scales[16] and an fp16 d, and
 *           each scale covers 16 consecutive weights (the corrected indexing
 *           the page documents; its bug gave one scale 32 weights).
 *   [PETIT] "PETIT — a tiny, CPU-first, quantized LLM inference engine"
 *           (README), "What makes it fast & small" and "How the pieces
 *           match": q8_0 = fp32 scale + 32 int8; q4_0 = fp16 scale + 16 bytes
 *           of 4-bit nibbles (18 bytes per 32 weights); weights are stored
 *           out x in and padded to whole 32-weight blocks.
 *   [S21v]  "picoLM, in Python", "§2 — K-quants", part "Verify against the
 *           spec, because even the C can be wrong": Q2_K is 84 bytes per
 *           256 weights (2.62 bits/weight), and the ggml specification is
 *           the formats' source of truth; "Exercises" item 2 names Q5_K and
 *           Q5_1. The pages give none of the byte layouts of Q2_K, Q3_K,
 *           Q5_K, Q5_1 or GGUF's Q8_0: those below are the ggml
 *           specification's, written out from it (a reading, see below).
 *
 * Readings where the pages leave a step open (each is listed in the design
 * notes of the repository):
 *   - Q6_K bit placement: weight 128h + 32k + l (h = half, k = quarter,
 *     l = 0..31) takes its low 4 bits from ql[64h + 32(k&1) + l] (low nibble
 *     for k < 2, high nibble for k >= 2) and its high 2 bits from bits 2k,2k+1
 *     of qh[32h + l]; the code is stored with an offset of 32. This is ggml's
 *     layout, which [S21] names as the format's source of truth.
 *   - q4_0 nibble order: byte j carries weight j (low nibble) and weight j+16
 *     (high nibble); value = d * (nibble - 8) (ggml's q4_0).
 *   - All multi-byte fields are little-endian.
 *   - Q8_0 with an fp16 scale (GGUF's Q8_0, 34 bytes): fp16 d, 32 int8;
 *     weight = d * q.
 *   - Q5_1 (24 bytes / 32): fp16 d, fp16 m, a little-endian uint32 of high
 *     bits, 16 nibble bytes; weight j < 16 is the low nibble of byte j with
 *     high-bit word bit j, weight j + 16 the high nibble with bit j + 16;
 *     weight = q * d + m (q = 0..31).
 *   - Q5_K (176 bytes / 256): Q4_K's header and packed scales (fp16 d, fp16
 *     dmin, 12 bytes), then qh[32], then 128 nibble bytes; weight 64g + l
 *     (low nibble of byte 32g + l) takes bit 2g of qh[l] as its fifth bit,
 *     weight 64g + 32 + l (high nibble) bit 2g + 1; weight =
 *     d*scale*q - dmin*min per 32-weight sub-block, as Q4_K.
 *   - Q2_K (84 bytes / 256): 16 scale bytes (low nibble scale, high nibble
 *     min, one byte per 16 weights), 64 code bytes, fp16 d, fp16 dmin.
 *     Weight 128h + 32j + l takes bits 2j..2j+1 of code byte 32h + l and
 *     scale byte (128h + 32j + l) / 16; weight = d*scale*q - dmin*min.
 *   - Q3_K (110 bytes / 256): hmask[32], 64 code bytes, 12 bytes of sixteen
 *     packed 6-bit scales, fp16 d. Weight 128h + 32j + l: low 2 bits = bits
 *     2j..2j+1 of code byte 32h + l, and the code is that minus 4 unless bit
 *     4h + j of hmask[l] is set; scale s = weight / 16 has its low 4 bits in
 *     byte s (low nibble, s < 8) or byte s - 8 (high nibble), its top 2 bits
 *     at bits 2(s/4)..2(s/4)+1 of byte 8 + s%4, and is stored plus 32;
 *     weight = d*(scale)*q.
 *
 * Precision: the pages fix the dequantised weights as fp32 ([S21] computes in
 * float32 NumPy arrays, [Q6K] in C float), so every dequantised weight is an
 * fp32 value computed in the pages' operation order, with no contraction
 * (-ffp-contract=off). GEMV/GEMM sums are taken in fp64, sequentially, as
 * the plain definition y[r] = sum_c w[r][c] * x[c].
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off -fPIC -shared -o libqk_oracle.so qk_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Format ids. The GPU library's ids have the same values; both sides define
 * them independently. */
enum { ORC_Q4_0 = 1, ORC_Q8_0 = 2, ORC_Q4_K = 3, ORC_Q6_K = 4,
       ORC_Q8_0_F16 = 5, ORC_Q5_1 = 6, ORC_Q5_K = 7, ORC_Q2_K = 8, ORC_Q3_K = 9 };

/* Bytes per block and weights per block, written from the pages' byte counts:
 * Q4_K 2+2+12+128 = 144 for 256 [S21]; Q6_K 128+64+16+2 = 210 for 256 [Q6K];
 * q4_0 2+16 = 18 for 32 and q8_0 4+32 = 36 for 32 [PETIT]. */
_Static_assert(2 + 2 + 12 + 128 == 144, "Q4_K block is 144 bytes");
_Static_assert(128 + 64 + 16 + 2 == 210, "Q6_K block is 210 bytes");
_Static_assert(2 + 16 == 18, "q4_0 block is 18 bytes");
_Static_assert(4 + 32 == 36, "q8_0 block is 36 bytes");
/* The ggml formats: Q2_K 16+64+2+2 = 84 [S21v]; Q3_K 32+64+12+2 = 110;
 * Q5_K 2+2+12+32+128 = 176; Q5_1 2+2+4+16 = 24; GGUF Q8_0 2+32 = 34. */
_Static_assert(16 + 64 + 2 + 2 == 84, "Q2_K block is 84 bytes");
_Static_assert(32 + 64 + 12 + 2 == 110, "Q3_K block is 110 bytes");
_Static_assert(2 + 2 + 12 + 32 + 128 == 176, "Q5_K block is 176 bytes");
_Static_assert(2 + 2 + 4 + 16 == 24, "Q5_1 block is 24 bytes");
_Static_assert(2 + 32 == 34, "fp16-scale Q8_0 block is 34 bytes");

int qko_block_elems(int type) {
    switch (type) {
    case ORC_Q4_K: case ORC_Q6_K: case ORC_Q5_K: case ORC_Q2_K: case ORC_Q3_K: return 256;
    case ORC_Q4_0: case ORC_Q8_0: case ORC_Q8_0_F16: case ORC_Q5_1: return 32;
    default: return -1;
    }
}

int qko_block_bytes(int type) {
    switch (type) {
    case ORC_Q4_K: return 2 + 2 + 12 + 128;
    case ORC_Q6_K: return 128 + 64 + 16 + 2;
    case ORC_Q4_0: return 2 + 16;
    case ORC_Q8_0: return 4 + 32;
    case ORC_Q8_0_F16: return 2 + 32;
    case ORC_Q5_1: return 2 + 2 + 4 + 16;
    case ORC_Q5_K: return 2 + 2 + 12 + 32 + 128;
    case ORC_Q2_K: return 16 + 64 + 2 + 2;
    case ORC_Q3_K: return 32 + 64 + 12 + 2;
    default: return -1;
    }
}

/* ---- scalar fields ----------------------------------------------------- */

static uint16_t rd_u16le(const uint8_t *p) { return (uint16_t)(p[0] | (p[1] << 8)); }

static uint32_t rd_u32le(const uint8_t *p) {
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

/* IEEE 754 binary16 -> binary32 from the fields: 1 sign bit, 5 exponent bits
 * (bias 15), 10 fraction bits. Subnormals are f * 2^-24; exponent 31 is
 * Inf/NaN. Exact: every binary16 value is representable in binary32. */
float qko_half_to_float(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1F;
    const int f = h & 0x3FF;
    float v;
    if (e == 0) {
        v = ldexpf((float)f, -24);
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexpf((float)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* bfloat16 is the top half of a binary32. */
float qko_bf16_to_float(uint16_t h) {
    const uint32_t u = (uint32_t)h << 16;
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
}

static float f32_from_bits(uint32_t u) {
    float v;
    memcpy(&v, &u, sizeof v);
    return v;
}

/* ---- block decoders ---------------------------------------------------- */

/* The 12 packed bytes shared by Q4_K and Q5_K hold sixteen 6-bit fields:
 * the scale and the min of each of the eight 32-weight sub-blocks ([S21] §2;
 * the fields of sub-blocks 4..7 straddle byte boundaries). Byte map, bit 0 =
 * least significant:
 *   bytes 0..3   bits 0..5: scale of sub-block 0..3;
 *                bits 6..7: top 2 bits of the scale of sub-block 4..7;
 *   bytes 4..7   bits 0..5: min of sub-block 0..3;
 *                bits 6..7: top 2 bits of the min of sub-block 4..7;
 *   bytes 8..11  bits 0..3: low 4 bits of the scale of sub-block 4..7;
 *                bits 4..7: low 4 bits of the min of sub-block 4..7.
 * A field is read as runs of the 96-bit little-endian bit string. */
static int packed_bits(const uint8_t *p, int bit, int width) {
    int v = 0;
    for (int i = 0; i < width; i++) v |= ((p[(bit + i) / 8] >> ((bit + i) % 8)) & 1) << i;
    return v;
}

static int k4_field(const uint8_t *packed, int is_min, int j) {
    const int first = is_min ? 32 : 0; /* bit 0 of bytes 0..3 (scales) or 4..7 (mins) */
    if (j < 4) return packed_bits(packed, first + 8 * j, 6);
    const int low4 = packed_bits(packed, 64 + 8 * (j - 4) + (is_min ? 4 : 0), 4);
    const int top2 = packed_bits(packed, first + 8 * (j - 4) + 6, 2);
    return low4 | (top2 << 4);
}

static void k4_scale_min(const uint8_t *packed, int j, int *s, int *m) {
    *s = k4_field(packed, 0, j);
    *m = k4_field(packed, 1, j);
}

/* [S21] §2: d at byte 0, dmin at byte 2, the 12 packed scale/min bytes at
 * 4..15, the 128 nibble bytes at 16..143. Sub-blocks j = 0..3 keep their
 * 6-bit scale and min in the low bits of their own bytes; sub-blocks 4..7
 * straddle: low 4 bits from byte j+4 (scale: low nibble, min: high nibble),
 * high 2 bits from the top of byte j-4 (scale) or byte j (min). Nibble byte
 * 32g + l gives weight 64g + l (low nibble, sub-block 2g) and weight
 * 64g + 32 + l (high nibble, sub-block 2g+1); each weight is
 * d*scale*q - dmin*min, evaluated left to right in fp32. */
static void decode_q4_K(const uint8_t *blk, float *out) {
    const float d = qko_half_to_float(rd_u16le(blk + 0));
    const float dmin = qko_half_to_float(rd_u16le(blk + 2));
    const uint8_t *packed = blk + 4;
    const uint8_t *qs = blk + 16;

    float sc[8], mn[8];
    for (int j = 0; j < 8; j++) {
        int s, m;
        k4_scale_min(packed, j, &s, &m);
        sc[j] = (float)s;
        mn[j] = (float)m;
    }

    for (int g = 0; g < 4; g++) {
        for (int half = 0; half < 2; half++) {
            const int j = 2 * g + half;
            for (int l = 0; l < 32; l++) {
                const uint8_t byte = qs[32 * g + l];
                const int q = half ? (byte >> 4) : (byte & 0xF);
                float t = d * sc[j];
                t = t * (float)q;
                const float m = dmin * mn[j];
                out[64 * g + 32 * half + l] = t - m;
            }
        }
    }
}

/* [Q6K] 原理: ql[128] at 0, qh[64] at 128, int8 scales[16] at 192, fp16 d at
 * 208. Weight i (h = i / 128, k = (i % 128) / 32, l = i % 32) has its low 4
 * bits in ql[64h + 32(k % 2) + l] (low nibble for k < 2, high nibble for
 * k >= 2) and its high 2 bits at bits 2k..2k+1 of qh[32h + l]; its code is
 * that 6-bit value minus 32. Each scale covers 16 consecutive weights, so
 * weight i takes scales[i / 16]. Weight = d * scale * q, left to right in
 * fp32. */
static void decode_q6_K(const uint8_t *blk, float *out) {
    const uint8_t *ql = blk;
    const uint8_t *qh = blk + 128;
    const int8_t *scales = (const int8_t *)(blk + 192);
    const float d = qko_half_to_float(rd_u16le(blk + 208));

    for (int i = 0; i < 256; i++) {
        const int h = i / 128, k = (i % 128) / 32, l = i % 32;
        const uint8_t lo_src = ql[64 * h + 32 * (k % 2) + l];
        const int low4 = (k < 2) ? (lo_src & 0xF) : (lo_src >> 4);
        const int high2 = (qh[32 * h + l] >> (2 * k)) & 3;
        const int q = (low4 | (high2 << 4)) - 32;
        float w = d * (float)scales[i / 16];
        w = w * (float)q;
        out[i] = w;
    }
}

/* [PETIT] q8_0: one fp32 scale, then 32 int8 values; weight = scale * q. */
static void decode_q8_0(const uint8_t *blk, float *out) {
    const float s = f32_from_bits(rd_u32le(blk));
    const int8_t *q = (const int8_t *)(blk + 4);
    for (int i = 0; i < 32; i++) out[i] = s * (float)q[i];
}

/* [PETIT] q4_0: one fp16 scale, then 16 bytes of nibbles. Reading: byte j
 * holds weight j (low nibble) and weight j+16 (high nibble), value
 * d * (nibble - 8). */
static void decode_q4_0(const uint8_t *blk, float *out) {
    const float d = qko_half_to_float(rd_u16le(blk));
    const uint8_t *qs = blk + 2;
    for (int j = 0; j < 16; j++) {
        out[j] = d * (float)((qs[j] & 0xF) - 8);
        out[j + 16] = d * (float)((qs[j] >> 4) - 8);
    }
}

/* GGUF's Q8_0 (reading, [S21v]): fp16 d at 0, int8 q[32] at 2; d * q. */
static void decode_q8_0_f16(const uint8_t *blk, float *out) {
    const float d = qko_half_to_float(rd_u16le(blk));
    const int8_t *q = (const int8_t *)(blk + 2);
    for (int i = 0; i < 32; i++) out[i] = d * (float)q[i];
}

/* Q5_1 (reading, [S21v]): fp16 d at 0, fp16 m at 2, uint32 qh at 4, 16
 * nibble bytes at 8. Byte j: low nibble = weight j with bit j of qh as its
 * fifth bit, high nibble = weight j + 16 with bit j + 16; q * d + m. */
static void decode_q5_1(const uint8_t *blk, float *out) {
    const float d = qko_half_to_float(rd_u16le(blk));
    const float m = qko_half_to_float(rd_u16le(blk + 2));
    const uint32_t qh = rd_u32le(blk + 4);
    const uint8_t *qs = blk + 8;
    for (int j = 0; j < 16; j++) {
        const int q0 = (qs[j] & 0xF) | (int)(((qh >> j) & 1u) << 4);
        const int q1 = (qs[j] >> 4) | (int)(((qh >> (j + 16)) & 1u) << 4);
        float t = (float)q0 * d;
        out[j] = t + m;
        t = (float)q1 * d;
        out[j + 16] = t + m;
    }
}

/* Q5_K (reading, [S21v]): Q4_K's header (d, dmin, 12 packed bytes) at 0,
 * qh[32] at 16, nibbles at 48. Nibble group g (bytes 32g..32g+31): the low
 * nibble of byte 32g + l is weight 64g + l of sub-block 2g, fifth bit = bit
 * 2g of qh[l]; the high nibble is weight 64g + 32 + l of sub-block 2g + 1,
 * fifth bit = bit 2g + 1 of qh[l]. Weight = d*scale*q - dmin*min. */
static void decode_q5_K(const uint8_t *blk, float *out) {
    const float d = qko_half_to_float(rd_u16le(blk + 0));
    const float dmin = qko_half_to_float(rd_u16le(blk + 2));
    const uint8_t *packed = blk + 4;
    const uint8_t *qh = blk + 16;
    const uint8_t *qs = blk + 48;
    for (int g = 0; g < 4; g++) {
        for (int half = 0; half < 2; half++) {
            const int j = 2 * g + half;
            int s, mn;
            k4_scale_min(packed, j, &s, &mn);
            for (int l = 0; l < 32; l++) {
                const uint8_t byte = qs[32 * g + l];
                const int low4 = half ? (byte >> 4) : (byte & 0xF);
                const int q = low4 | (((qh[l] >> j) & 1) << 4);
                float t = d * (float)s;
                t = t * (float)q;
                const float m = dmin * (float)mn;
                out[64 * g + 32 * half + l] = t - m;
            }
        }
    }
}

/* Q2_K (reading; size from [S21v]): scales[16] at 0 (low nibble = scale,
 * high nibble = min), qs[64] at 16, fp16 d at 80, fp16 dmin at 82. Half h
 * (128 weights) uses code bytes 32h..32h+31; its four 32-weight quarters j
 * take bits 2j, 2j+1 of those bytes. Each 16 weights share one scale byte.
 * Weight = d*scale*q - dmin*min. */
static void decode_q2_K(const uint8_t *blk, float *out) {
    const uint8_t *scales = blk;
    const uint8_t *qs = blk + 16;
    const float d = qko_half_to_float(rd_u16le(blk + 80));
    const float dmin = qko_half_to_float(rd_u16le(blk + 82));
    for (int h = 0; h < 2; h++) {
        for (int j = 0; j < 4; j++) {
            for (int l = 0; l < 32; l++) {
                const int i = 128 * h + 32 * j + l;
                const uint8_t sb = scales[i / 16];
                const int q = (qs[32 * h + l] >> (2 * j)) & 3;
                float t = d * (float)(sb & 0xF);
                t = t * (float)q;
                const float m = dmin * (float)(sb >> 4);
                out[i] = t - m;
            }
        }
    }
}

/* Q3_K (reading, [S21v]): hmask[32] at 0, qs[64] at 32, 12 packed scale
 * bytes at 96, fp16 d at 108. Weight 128h + 32j + l: q = bits 2j..2j+1 of
 * qs[32h + l], minus 4 unless bit 4h + j of hmask[l] is set. Scale
 * s = weight/16 is 6 bits: low 4 from byte s (s < 8, low nibble) or byte
 * s - 8 (high nibble), high 2 from bits 2(s/4), 2(s/4)+1 of byte 8 + s%4;
 * its value is that minus 32. Weight = d*scale*q. */
static void decode_q3_K(const uint8_t *blk, float *out) {
    const uint8_t *hmask = blk;
    const uint8_t *qs = blk + 32;
    const uint8_t *sp = blk + 96;
    const float d = qko_half_to_float(rd_u16le(blk + 108));
    int sc[16];
    for (int s = 0; s < 16; s++) {
        const int low4 = s < 8 ? (sp[s] & 0xF) : (sp[s - 8] >> 4);
        const int high2 = (sp[8 + s % 4] >> (2 * (s / 4))) & 3;
        sc[s] = (low4 | (high2 << 4)) - 32;
    }
    for (int h = 0; h < 2; h++) {
        for (int j = 0; j < 4; j++) {
            for (int l = 0; l < 32; l++) {
                const int i = 128 * h + 32 * j + l;
                const int q2 = (qs[32 * h + l] >> (2 * j)) & 3;
                const int hb = (hmask[l] >> (4 * h + j)) & 1;
                const int q = q2 - (hb ? 0 : 4);
                float w = d * (float)sc[i / 16];
                w = w * (float)q;
                out[i] = w;
            }
        }
    }
}

typedef void (*decode_fn)(const uint8_t *, float *);

static decode_fn decoder_for(int type) {
    switch (type) {
    case ORC_Q4_K: return decode_q4_K;
    case ORC_Q6_K: return decode_q6_K;
    case ORC_Q8_0: return decode_q8_0;
    case ORC_Q4_0: return decode_q4_0;
    case ORC_Q8_0_F16: return decode_q8_0_f16;
    case ORC_Q5_1: return decode_q5_1;
    case ORC_Q5_K: return decode_q5_K;
    case ORC_Q2_K: return decode_q2_K;
    case ORC_Q3_K: return decode_q3_K;
    default: return NULL;
    }
}

/* ---- public entry points ---------------------------------------------- */

/* Dequantise n weights (n a multiple of the block size) from consecutive
 * blocks into out[n] (fp32). The stand-in for the pages' dequantize_row(src,
 * dst, n, type) ([S21] §4, the token-embedding row). Returns 0 or -1. */
int qko_dequantize_row(int type, const void *blocks, int64_t n, float *out) {
    const decode_fn dec = decoder_for(type);
    const int qk = qko_block_elems(type);
    const int bb = qko_block_bytes(type);
    if (!dec || n < 0 || n % qk != 0 || (n > 0 && (!blocks || !out))) return -1;
    const uint8_t *src = (const uint8_t *)blocks;
    for (int64_t b = 0; b < n / qk; b++) dec(src + b * bb, out + b * qk);
    return 0;
}

/* y[r] = sum_c w[r][c] * x[c] in fp64, summed over c in order, where w[r][c]
 * is the fp32 dequantised weight; absacc[r] = sum_c |w[r][c] * x[c]| (the
 * tolerance scale). W is rows x (cols/QK) blocks, row-major, out x in
 * ([PETIT] "How the pieces match"; the matmul(out, x, W, n_in, n_out) calls
 * of [S21] §4). absacc may be NULL. Returns 0 or -1. */
int qko_gemv(int type, const void *W, int64_t rows, int64_t cols,
             const float *x, double *y, double *absacc) {
    const decode_fn dec = decoder_for(type);
    const int qk = qko_block_elems(type);
    const int bb = qko_block_bytes(type);
    if (!dec || rows < 0 || cols < 0 || cols % qk != 0) return -1;
    if (rows == 0 || cols == 0) {
        for (int64_t r = 0; r < rows; r++) { y[r] = 0.0; if (absacc) absacc[r] = 0.0; }
        return 0;
    }
    float *w = (float *)malloc((size_t)cols * sizeof(float));
    if (!w) return -1;
    const int64_t row_bytes = cols / qk * bb;
    for (int64_t r = 0; r < rows; r++) {
        qko_dequantize_row(type, (const uint8_t *)W + r * row_bytes, cols, w);
        double s = 0.0, a = 0.0;
        for (int64_t c = 0; c < cols; c++) {
            const double p = (double)w[c] * (double)x[c];
            s += p;
            a += fabs(p);
        }
        y[r] = s;
        if (absacc) absacc[r] = a;
    }
    free(w);
    return 0;
}

/* Y[m][r] = sum_c w[r][c] * X[m][c] for M activation rows X given in
 * bfloat16 ([M][cols], row-major), each widened to fp32 exactly; fp64 sums
 * as in qko_gemv. Y and absacc are [M][rows]. absacc may be NULL. */
int qko_gemm(int type, const void *W, int64_t rows, int64_t cols,
             const uint16_t *X, int64_t M, double *Y, double *absacc) {
    const decode_fn dec = decoder_for(type);
    const int qk = qko_block_elems(type);
    const int bb = qko_block_bytes(type);
    if (!dec || rows < 0 || cols < 0 || M < 0 || cols % qk != 0) return -1;
    float *w = (float *)malloc(((size_t)cols + 1) * sizeof(float));
    float *x = (float *)malloc(((size_t)M * (size_t)cols + 1) * sizeof(float));
    if (!w || !x) { free(w); free(x); return -1; }
    for (int64_t i = 0; i < M * cols; i++) x[i] = qko_bf16_to_float(X[i]);
    const int64_t row_bytes = cols / qk * bb;
    for (int64_t r = 0; r < rows; r++) {
        qko_dequantize_row(type, (const uint8_t *)W + r * row_bytes, cols, w);
        for (int64_t m = 0; m < M; m++) {
            const float *xm = x + m * cols;
            double s = 0.0, a = 0.0;
            for (int64_t c = 0; c < cols; c++) {
                const double p = (double)w[c] * (double)xm[c];
                s += p;
                a += fabs(p);
            }
            Y[m * rows + r] = s;
            if (absacc) absacc[m * rows + r] = a;
        }
    }
    free(w);
    free(x);
    return 0;
}

/* ==== the decode step around the GEMVs, and the encoder ==================
 *
 * Sources: [S21] §4 "The forward pass" (model_forward: dequantise the
 * token's embedding row; per layer RMSNorm, the q/k/v projections, RoPE on
 * q and k with the position's cos/sin, K and V stored in an fp16 cache at
 * `pos` — K after RoPE — attention of every query head over positions
 * 0..pos against the KV head it shares (n_kv_heads < n_heads), softmax,
 * output projection, SwiGLU, residuals; a final RMSNorm and the output
 * matrix); [S21] §3 "The RoPE layout is not the one you learned" (the
 * interleaved rotation of the pair (x[2i], x[2i+1]) by cos[i], sin[i]);
 * [PETIT] "What makes it fast & small" (RoPE + RMSNorm + SwiGLU) and "How the
 * pieces match" (RoPE base 10000, per head; the exporter quantises fp32
 * weights into q8_0 / q4_0 blocks).
 *
 * Readings (the pages leave these open):
 *   - RMSNorm: out_i = w_i * x_i / sqrt(mean(x^2) + eps), eps an argument.
 *   - RoPE frequencies: theta_i = base^(-2i/head_dim), angle = pos*theta_i.
 *   - Attention scale 1/sqrt(head_dim); query head h uses KV head
 *     h / (n_heads / n_kv_heads).
 *   - SwiGLU: silu(gate) * up with silu(g) = g / (1 + exp(-g)).
 *   - The quantiser rule (the pages give only the block formats): q8_0
 *     d = amax/127, q = round-half-away(x * (1/d)); q4_0 with m the value of
 *     largest magnitude, d = m / -8, q = min(15, trunc(x * (1/d) + 8.5)),
 *     stored scale fp16(d) — the ggml reference quantisers.
 *   - fp32 -> fp16 (the cache) rounds to nearest even.
 * Plain definitions in fp64 where the result is a real number (norm, RoPE,
 * attention, SwiGLU), rounded once to fp32 for outputs that are fp32 on the
 * path; the quantiser in fp32 operations in the stated order (its result is
 * an integer decided by those operations). */

/* IEEE 754 binary32 -> binary16, round to nearest, ties to even; overflow to
 * infinity, NaN kept NaN, subnormal results rounded at 2^-24. */
uint16_t qko_float_to_half(float f) {
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint32_t sign = (u >> 16) & 0x8000u;
    const int e = (int)((u >> 23) & 0xFF);
    const uint32_t m = u & 0x7FFFFFu;
    if (e == 255) return (uint16_t)(sign | 0x7C00u | (m ? 0x200u : 0u));
    const double a = fabs((double)f);
    if (a == 0.0) return (uint16_t)sign;
    /* scale so that one binary16 ulp at this magnitude is 1, round to even */
    int ex;
    frexp(a, &ex);                 /* a = fr * 2^ex, fr in [0.5, 1) */
    int ulp_exp = ex - 11;         /* ulp of a normal binary16 with this exponent */
    if (ulp_exp < -24) ulp_exp = -24;  /* subnormal range: ulp 2^-24 */
    const double scaled = ldexp(a, -ulp_exp);   /* exact (power-of-two scale) */
    double r = floor(scaled);
    const double frac = scaled - r;
    if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    const double v = ldexp(r, ulp_exp);       /* the rounded magnitude */
    if (v > 65504.0) return (uint16_t)(sign | 0x7C00u);
    /* encode v */
    if (v < ldexp(1.0, -14)) return (uint16_t)(sign | (uint32_t)ldexp(v, 24));
    int ve;
    const double vf = frexp(v, &ve);          /* v = vf * 2^ve, vf in [0.5, 1) */
    const uint32_t hexp = (uint32_t)(ve - 1 + 15);
    const uint32_t hman = (uint32_t)ldexp(vf * 2.0 - 1.0, 10);
    return (uint16_t)(sign | (hexp << 10) | hman);
}

/* out_i = w_i * x_i / sqrt(mean(x^2) + eps), in fp64, rounded to fp32. */
void qko_rmsnorm(const float *x, const float *w, int64_t n, float eps, float *out) {
    double ss = 0.0;
    for (int64_t i = 0; i < n; i++) ss += (double)x[i] * (double)x[i];
    const double inv = 1.0 / sqrt(ss / (double)n + (double)eps);
    for (int64_t i = 0; i < n; i++) out[i] = (float)((double)w[i] * ((double)x[i] * inv));
}

/* cos/sin of pos * theta_i, theta_i = base^(-2i/head_dim), i < head_dim/2,
 * in fp64, rounded to fp32. */
void qko_rope_table(int64_t pos, int head_dim, double base, float *c, float *s) {
    for (int i = 0; i < head_dim / 2; i++) {
        const double theta = pow(base, -2.0 * (double)i / (double)head_dim);
        const double ang = (double)pos * theta;
        c[i] = (float)cos(ang);
        s[i] = (float)sin(ang);
    }
}

/* [S21] §3: per head, the pair (x[2i], x[2i+1]) becomes
 * (x0*cos[i] - x1*sin[i], x0*sin[i] + x1*cos[i]); fp64, rounded to fp32. */
void qko_rope_interleaved(float *x, int n_heads, int head_dim, const float *c, const float *s) {
    for (int h = 0; h < n_heads; h++) {
        float *v = x + (int64_t)h * head_dim;
        for (int i = 0; i < head_dim / 2; i++) {
            const double x0 = v[2 * i], x1 = v[2 * i + 1];
            v[2 * i] = (float)(x0 * (double)c[i] - x1 * (double)s[i]);
            v[2 * i + 1] = (float)(x0 * (double)s[i] + x1 * (double)c[i]);
        }
    }
}

/* Attention of one position's queries over the fp16 cache: for query head
 * h, KV head g = h / (n_heads / n_kv), scores_t = (K[t, g] . q_h) /
 * sqrt(head_dim) for t < n_pos, p = softmax(scores) (max-subtracted, two
 * passes), out_h = sum_t p_t V[t, g]. Cache rows are kv_stride halves apart
 * (row t, head g at t*kv_stride + g*head_dim). fp64 throughout; absacc_h,i =
 * sum_t p_t |V[t, g, i]| (a tolerance scale). */
void qko_attention(const float *q, const uint16_t *kc, const uint16_t *vc, int n_heads, int n_kv, int head_dim,
                   int64_t n_pos, int64_t kv_stride, double *out, double *absacc) {
    const int grp = n_heads / n_kv;
    const double scale = 1.0 / sqrt((double)head_dim);
    double *sc = (double *)malloc((size_t)(n_pos > 0 ? n_pos : 1) * sizeof(double));
    if (!sc) return;
    for (int h = 0; h < n_heads; h++) {
        const int g = h / grp;
        const float *qh = q + (int64_t)h * head_dim;
        double mx = -INFINITY;
        for (int64_t t = 0; t < n_pos; t++) {
            const uint16_t *k = kc + t * kv_stride + (int64_t)g * head_dim;
            double dot = 0.0;
            for (int i = 0; i < head_dim; i++) dot += (double)qko_half_to_float(k[i]) * (double)qh[i];
            sc[t] = dot * scale;
            if (sc[t] > mx) mx = sc[t];
        }
        double sum = 0.0;
        for (int64_t t = 0; t < n_pos; t++) {
            sc[t] = exp(sc[t] - mx);
            sum += sc[t];
        }
        for (int i = 0; i < head_dim; i++) {
            double acc = 0.0, aa = 0.0;
            for (int64_t t = 0; t < n_pos; t++) {
                const double v = (double)qko_half_to_float(vc[t * kv_stride + (int64_t)g * head_dim + i]);
                acc += sc[t] * v;
                aa += sc[t] * fabs(v);
            }
            out[(int64_t)h * head_dim + i] = acc / sum;
            if (absacc) absacc[(int64_t)h * head_dim + i] = aa / sum;
        }
    }
    free(sc);
}

/* silu(g) * u = g * u / (1 + exp(-g)), fp64. */
void qko_swiglu(const float *g, const float *u, int64_t n, double *out) {
    for (int64_t i = 0; i < n; i++) {
        const double gv = g[i];
        out[i] = gv / (1.0 + exp(-gv)) * (double)u[i];
    }
}

/* The encoder: fp32 weights -> blocks (n a multiple of 32). q8_0: amax over
 * the block, d = amax / 127, id = 1/d (0 when d = 0), q_j = round-half-away
 * (x_j * id), stored as fp32 d and int8 q. q4_0: m = the value of largest
 * magnitude (the first such), d = m / -8, id = 1/d (0 when d = 0), code =
 * min(15, trunc(x_j * id + 8.5)), weight j in the low nibble of byte j and
 * weight j + 16 in the high nibble, stored scale fp16(d). Every operation is
 * one fp32 operation, rounded to nearest even, in this order. Returns 0 or
 * -1. */
int qko_quantize(int type, const float *x, int64_t n, void *blocks) {
    if ((type != ORC_Q8_0 && type != ORC_Q4_0) || n < 0 || n % 32 != 0) return -1;
    uint8_t *dst = (uint8_t *)blocks;
    for (int64_t b = 0; b < n / 32; b++) {
        const float *v = x + b * 32;
        if (type == ORC_Q8_0) {
            float amax = 0.0f;
            for (int j = 0; j < 32; j++) {
                const float a = fabsf(v[j]);
                if (a > amax) amax = a;
            }
            const float d = amax / 127.0f;
            const float id = d != 0.0f ? 1.0f / d : 0.0f;
            uint8_t *blk = dst + b * 36;
            memcpy(blk, &d, 4);
            for (int j = 0; j < 32; j++) {
                const float t = v[j] * id;
                blk[4 + j] = (uint8_t)(int8_t)roundf(t);
            }
        } else {
            float amax = 0.0f, m = 0.0f;
            for (int j = 0; j < 32; j++) {
                const float a = fabsf(v[j]);
                if (a > amax) {
                    amax = a;
                    m = v[j];
                }
            }
            const float d = m / -8.0f;
            const float id = d != 0.0f ? 1.0f / d : 0.0f;
            uint8_t *blk = dst + b * 18;
            const uint16_t dh = qko_float_to_half(d);
            blk[0] = (uint8_t)(dh & 0xFF);
            blk[1] = (uint8_t)(dh >> 8);
            for (int j = 0; j < 16; j++) {
                const float t0 = v[j] * id + 8.5f;
                const float t1 = v[j + 16] * id + 8.5f;
                int c0 = (int)t0, c1 = (int)t1; /* t0, t1 in [0.5, 16.5]: truncation */
                if (c0 > 15) c0 = 15;
                if (c1 > 15) c1 = 15;
                blk[2 + j] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
    return 0;
}
