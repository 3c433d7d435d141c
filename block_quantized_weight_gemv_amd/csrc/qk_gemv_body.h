// qk_gemv_body.h — the fused dequantise-and-dot GEMV, y = W x (M = 1): the
// device code shared by the per-stage launches (qk_gemv.hip) and the
// persistent decode pass (qk_pass.hip).
//
// The pages' matmul walks the quantised bytes and accumulates the dot product
// as it decodes, so only the packed weights cross the memory bus ("picoLM, in
// Python", §3 Tensor ops; the fused vec_dot of "PicoLM Q6_K量化Bug调试全记录").
// This is that loop laid out for a 64-wide CDNA4 wavefront:
//
// * A lane owns one "unit" of a row: 64 weights of a K-quant block (Q4_K: one
//   32-byte nibble group = sub-blocks 2g and 2g+1; Q6_K: one 16-position
//   column of a 128-weight half = four 16-weight scale groups) or one whole
//   32-weight q8_0/q4_0 block. The lane keeps x for its unit in VGPRs, plus
//   the sums of x over each scale group, for every row it visits: x is read
//   once per wave, not once per row.
// * A row's units sit in adjacent lanes, so the packed bytes of a row are read
//   with 16-byte loads by neighbouring lanes (coalesced, every byte once).
//   Rows with at most 32 units share a wave (2, 4, ... rows per wave step);
//   rows with more than 64 units are split over 2-8 waves of a workgroup and
//   combined in LDS in a fixed order (deterministic).
// * Integer codes are converted with v_cvt_f32_ubyte on byte-masked words
//   and multiplied into fp32 accumulators; block scales are applied once per
//   scale group in factored form:
//     Q4_K  d*(sc0*S0 + sc1*S1) - dmin*(mn0*X0 + mn1*X1)
//     Q6_K  d*sum_k sc_k*(S_k - 32*X_k)
//     Q8_0  s*(S - 128*X)   (codes read as unsigned q+128)
//     Q4_0  d*(S - 8*X)
//   where S are sums of unsigned codes times x and X are sums of x. The
//   4-bit codes of Q4_K and q4_0 are converted two per instruction
//   (v_cvt_pk_f32_fp8, exact for 0..15), the others one per instruction.
// * Lane partials are reduced with a butterfly inside the row's lanes; one
//   lane writes y[r].
//
// * Large launches (>= 128 MiB, rows that one wave covers) stream each group
//   of consecutive rows through LDS instead: the workgroup reads the group's
//   bytes as one contiguous run of 16-byte pieces with the streaming cache
//   policy, so that every load instruction covers whole cache lines, and the
//   lanes read their units from the LDS copy. (With loads shaped like the
//   units, pieces of one cache line come from several instructions, and the
//   streaming policy would fetch such lines more than once.)
//
// Q6_K (210-byte) and q4_0 (18-byte) blocks are only 2-byte aligned. With an
// even number of blocks per row every row starts 4-byte aligned, and each
// piece is read as aligned dwords from the 4-byte boundary below it and
// realigned with v_alignbyte_b32; every such window stays inside the block
// pair (for Q3_K a window may end 2 bytes into the next block, so odd block
// counts need an even row count; Q6_K reads its last four bytes as two 2-byte
// loads; q4_0 needs an even block count).
// Rows wider than 6144 columns run the wide-row kernel (x staged in
// batches, up to 512 units over up to 8 waves); the shapes the fused kernels
// do not take use the generic kernel (qk_gemv.hip).
#pragma once

#include "qk_decode.h"
#include "qk_launch.h"

namespace qk {

template <int F> struct Unit;
template <> struct Unit<Q4_K> { static constexpr int W = 64, NSUM = 2; };
template <> struct Unit<Q6_K> { static constexpr int W = 64, NSUM = 4; };
template <> struct Unit<Q8_0> { static constexpr int W = 32, NSUM = 1; };
template <> struct Unit<Q4_0> { static constexpr int W = 32, NSUM = 1; };
template <> struct Unit<Q5_K> { static constexpr int W = 64, NSUM = 2; };       // as Q4_K
template <> struct Unit<Q2_K> { static constexpr int W = 64, NSUM = 4; };       // as Q6_K
template <> struct Unit<Q3_K> { static constexpr int W = 64, NSUM = 4; };       // as Q6_K
template <> struct Unit<Q5_1> { static constexpr int W = 32, NSUM = 1; };       // one block
template <> struct Unit<Q8_0_F16> { static constexpr int W = 32, NSUM = 1; };   // one block

template <int F> struct XUnit {
    float v[Unit<F>::W];
    float s[Unit<F>::NSUM];
};

// How the lanes of a workgroup cover rows; it depends only on the width and
// the unit size, so Q4_K and Q6_K (and q4_0 and q8_0) share it.
struct GemvPlan {
    int U;       // units per row
    int KS;      // waves that split one row's units
    int Uw;      // units per wave segment
    int Lshift;  // log2(lanes per row slot)
    int RP;      // row slots per wave
    int NWR;     // row waves per workgroup
    int ksmul;   // 65536 / KS + 1: (wave * ksmul) >> 16 == wave / KS for wave < 4
};

__device__ __forceinline__ void load4(const float *p, float *d) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
}

// x is staged once per workgroup in LDS: float f of x sits at position
// f + 4*(f/64) (4 floats of padding per 64, so that lanes reading 64-float
// units at a 68-float stride hit distinct banks), followed by the sums of x
// over each aligned group of 16 floats. Each lane then copies its unit's x
// and the sums it needs into registers.
__device__ __forceinline__ int xpos(int f) { return f + 4 * (f >> 6); }

__device__ __forceinline__ void lds4(const float *p, float *d) {
    const float4 v = *reinterpret_cast<const float4 *>(p);
    d[0] = v.x;
    d[1] = v.y;
    d[2] = v.z;
    d[3] = v.w;
}

// Three unit shapes:
//   W = 64, NSUM = 2 (Q4_K, Q5_K): weights 64g .. 64g+63 of a block, with
//     the sums of x over its two 32-weight sub-blocks;
//   W = 64, NSUM = 4 (Q6_K, Q2_K, Q3_K): 16 positions l0 .. l0+15 of each
//     of the four 32-weight quarters of a 128-weight half, with the sum of
//     x over each 16 (one scale group each);
//   W = 32 (Q8_0, Q4_0, Q5_1, Q8_0_F16): one block, with the sum of its x.
template <int F> __device__ __forceinline__ void read_x(const float *xs, const float *xsum, int u, XUnit<F> &xu) {
    if constexpr (Unit<F>::W == 64 && Unit<F>::NSUM == 2) {
        const float *p = xs + xpos(64 * u);  // block u/4, group u%4: weights 64g .. 64g+63
#pragma unroll
        for (int i = 0; i < 64; i += 4) lds4(p + i, xu.v + i);
        xu.s[0] = xsum[4 * u] + xsum[4 * u + 1];
        xu.s[1] = xsum[4 * u + 2] + xsum[4 * u + 3];
    } else if constexpr (Unit<F>::W == 64) {
        const int b = u >> 2, h = (u >> 1) & 1, l0 = 16 * (u & 1);
        const int f0 = 256 * b + 128 * h + l0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const float *p = xs + xpos(f0 + 32 * k);
#pragma unroll
            for (int t = 0; t < 16; t += 4) lds4(p + t, xu.v + 16 * k + t);
            xu.s[k] = xsum[(f0 + 32 * k) >> 4];
        }
    } else {
        const float *p = xs + xpos(32 * u);
#pragma unroll
        for (int i = 0; i < 32; i += 4) lds4(p + i, xu.v + i);
        xu.s[0] = xsum[2 * u] + xsum[2 * u + 1];
    }
}

__device__ __forceinline__ float byte_f(uint32_t w, int k) { return (float)((w >> (8 * k)) & 0xFFu); }

// Sum over the 4 bytes of w (unsigned) times 4 x values. The empty asm hides
// the bits of w from the compiler: when it can see that a byte holds a
// nibble it converts each byte with v_bfe_u32 + v_cvt_f32_ubyte0 (two ops)
// instead of one v_cvt_f32_ubyte{0..3}.
__device__ __forceinline__ float dot4u(uint32_t w, const float *xv, float acc) {
    __asm__("" : "+v"(w));
    acc += byte_f(w, 0) * xv[0];
    acc += byte_f(w, 1) * xv[1];
    acc += byte_f(w, 2) * xv[2];
    acc += byte_f(w, 3) * xv[3];
    return acc;
}

// Sum over the 4 bytes of w, each a nibble value 0..15, times 4 x values,
// all scaled by 2^-9: read as OCP E4M3 fp8, bytes 0..15 are exactly
// b * 2^-9 (0..7 subnormal, 8..15 the first binade), so v_cvt_pk_f32_fp8
// converts two codes per instruction. The caller multiplies the group sum
// by 512 (exact).
__device__ __forceinline__ float dot4_nib(uint32_t w, const float *xv, float acc) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
    acc += lo[0] * xv[0];
    acc += lo[1] * xv[1];
    acc += hi[0] * xv[2];
    acc += hi[1] * xv[3];
    return acc;
}

// Raw bytes of one unit of one row, loaded ahead of use so that the next
// row's loads are in flight while the current row is decoded.
template <int F> struct Raw;
template <> struct Raw<Q4_K> { u32x4 h, qa, qb; };
template <> struct Raw<Q6_K> { u32x4 p[3]; u32x4 s; uint32_t s4, e[3]; };  // s4: q6k_tail; e: each piece's next dword
template <> struct Raw<Q8_0> { uint32_t sc; u32x4 qa, qb; };
template <> struct Raw<Q4_0> { u32x4 w; uint32_t w4; };
template <> struct Raw<Q5_K> { u32x4 h, qa, qb, ha, hb; };
template <> struct Raw<Q2_K> { u32x4 q; u32x2 s; uint32_t dd; };
template <> struct Raw<Q3_K> { u32x4 hm, q, s; uint32_t hm4, q4; };
template <> struct Raw<Q5_1> { u32x2 h; u32x4 q; };
template <> struct Raw<Q8_0_F16> { u32x4 a, b; uint32_t c; };

template <int F> __device__ __forceinline__ void load_raw(const uint8_t *__restrict__ row, int u, Raw<F> &r);
// Partial dot product of unit u of a row (its raw bytes in r) with x.
template <int F> __device__ __forceinline__ float dot_raw(const uint8_t *__restrict__ row, int u, const Raw<F> &r,
                                                          const XUnit<F> &xu);

template <> __device__ __forceinline__ void load_raw<Q4_K>(const uint8_t *__restrict__ row, int u, Raw<Q4_K> &r) {
    const uint8_t *blk = row + (u >> 2) * 144;
    const int g = u & 3;
    r.h = ld_b128(blk);  // d|dmin, packed 0..3, 4..7, 8..11
    r.qa = ld_b128(blk + 16 + 32 * g);
    r.qb = ld_b128(blk + 32 + 32 * g);
}

template <> __device__ __forceinline__ float dot_raw<Q4_K>(const uint8_t *__restrict__, int u, const Raw<Q4_K> &r,
                                                           const XUnit<Q4_K> &xu) {
    const int g = u & 3;
    const uint32_t q[8] = {r.qa.x, r.qa.y, r.qa.z, r.qa.w, r.qb.x, r.qb.y, r.qb.z, r.qb.w};
    float s0 = 0.f, s1 = 0.f;  // both scaled by 2^-9
#pragma unroll
    for (int i = 0; i < 8; i++) {
        s0 = dot4_nib(q[i] & 0x0F0F0F0Fu, xu.v + 4 * i, s0);                // low nibbles: sub-block 2g
        s1 = dot4_nib((q[i] >> 4) & 0x0F0F0F0Fu, xu.v + 32 + 4 * i, s1);  // high nibbles: sub-block 2g+1
    }
    const u32x4 h = r.h;
    // Six-bit scales/mins of all eight sub-blocks, one per byte.
    const uint32_t sc_lo = h.y & 0x3F3F3F3Fu;
    const uint32_t mn_lo = h.z & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t mn_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    const uint32_t SC = g < 2 ? sc_lo : sc_hi;
    const uint32_t MN = g < 2 ? mn_lo : mn_hi;
    const int sh = 16 * (g & 1);
    const float sc0 = (float)((SC >> sh) & 0xFFu), sc1 = (float)((SC >> (sh + 8)) & 0xFFu);
    const float mn0 = (float)((MN >> sh) & 0xFFu), mn1 = (float)((MN >> (sh + 8)) & 0xFFu);
    const float d = half_bits_to_float(h.x & 0xFFFFu);
    const float dmin = half_bits_to_float(h.x >> 16);
    const float a = sc0 * s0 + sc1 * s1;
    const float m = mn0 * xu.s[0] + mn1 * xu.s[1];
    return (d * 512.f) * a - dmin * m;
}

__device__ __forceinline__ const uint8_t *q6k_block(const uint8_t *row, int u, uint32_t &mis) {
    const uint8_t *B0 = row + (u >> 2) * 210;
    mis = (uint32_t)(uintptr_t)B0 & 3u;  // 0 (even block) or 2 (odd block)
    return B0 - mis;                     // 4-byte aligned base of the block's windows
}

template <> __device__ __forceinline__ void load_raw<Q6_K>(const uint8_t *__restrict__ row, int u, Raw<Q6_K> &r) {
    const int h = (u >> 1) & 1, l0 = 16 * (u & 1);
    uint32_t mis;
    const uint8_t *A0 = q6k_block(row, u, mis);
    r.p[0] = ld_b128(A0 + 64 * h + l0);        // ql, quarters 0 and 2
    r.p[1] = ld_b128(A0 + 64 * h + 32 + l0);   // ql, quarters 1 and 3
    r.p[2] = ld_b128(A0 + 128 + 32 * h + l0);  // qh
    r.s = ld_b128(A0 + 192);                   // scales
    r.s4 = q6k_tail(A0 + mis);                 // scales 14, 15 and d
    // the dword after each piece (inside the block: the last ends at byte
    // 196 of the aligned-down block), for the realignment of a block that
    // starts 2 bytes past a 4-byte boundary
    r.e[0] = ld_b32(A0 + 64 * h + l0 + 16);
    r.e[1] = ld_b32(A0 + 64 * h + 32 + l0 + 16);
    r.e[2] = ld_b32(A0 + 128 + 32 * h + l0 + 16);
}

// lane i receives v from lane i+N (SHL) or i-N (SHR) of its 16-lane row.
template <int CTRL> __device__ __forceinline__ uint32_t dpp_mov(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_SHL1 = 0x101, DPP_SHR1 = 0x111, DPP_SHR3 = 0x113;

template <> __device__ __forceinline__ float dot_raw<Q6_K>(const uint8_t *__restrict__ row, int u, const Raw<Q6_K> &r,
                                                           const XUnit<Q6_K> &xu) {
    const int v = u & 3, h = v >> 1, l0 = 16 * (v & 1);
    uint32_t mis;
    (void)q6k_block(row, u, mis);
    // Each 16-byte piece starts at the 4-byte boundary at or below its
    // address; when the block is misaligned by 2 the piece needs one more
    // dword, loaded with it (e). (Taking that dword from the neighbouring
    // lane that loads it as its first, with DPP and selects, costs 13 VALU
    // operations per unit in a loop bound by VALU issue; the load costs
    // none.)
    const uint32_t ext[3] = {r.e[0], r.e[1], r.e[2]};
    uint32_t P[3][4];
#pragma unroll
    for (int pc = 0; pc < 3; pc++) {
        const u32x4 w = r.p[pc];
        P[pc][0] = align_bytes(w.y, w.x, mis);
        P[pc][1] = align_bytes(w.z, w.y, mis);
        P[pc][2] = align_bytes(w.w, w.z, mis);
        P[pc][3] = align_bytes(ext[pc], w.w, mis);
    }
    float S[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t A = P[0][i], B = P[1][i], H = P[2][i];
        const uint32_t c0 = (A & 0x0F0F0F0Fu) | ((H << 4) & 0x30303030u);
        const uint32_t c1 = (B & 0x0F0F0F0Fu) | ((H << 2) & 0x30303030u);
        const uint32_t c2 = ((A >> 4) & 0x0F0F0F0Fu) | (H & 0x30303030u);
        const uint32_t c3 = ((B >> 4) & 0x0F0F0F0Fu) | ((H >> 2) & 0x30303030u);
        S[0] = dot4u(c0, xu.v + 0 + 4 * i, S[0]);
        S[1] = dot4u(c1, xu.v + 16 + 4 * i, S[1]);
        S[2] = dot4u(c2, xu.v + 32 + 4 * i, S[2]);
        S[3] = dot4u(c3, xu.v + 48 + 4 * i, S[3]);
    }
    // scales 8h..8h+3 and 8h+4..8h+7 of this half; this unit uses bytes
    // l0/16 + {0, 2} of each (quarters k = 0,1 and k = 2,3).
    // (a misaligned block's scale window ends at byte 205: its scales 14
    // and 15 are the low half of the tail dword, which is then also the
    // dword after the window)
    const u32x4 s = r.s;
    const uint32_t lo0 = h ? s.z : s.x, hi0 = h ? s.w : s.y, hi1 = h ? r.s4 : s.z;
    const uint32_t SC0 = align_bytes(hi0, lo0, mis);
    const uint32_t SC1 = align_bytes(hi1, hi0, mis);
    const int sb = 8 * (l0 >> 4);
    const float sc0 = (float)(int)(int8_t)(SC0 >> sb);
    const float sc1 = (float)(int)(int8_t)(SC0 >> (16 + sb));
    const float sc2 = (float)(int)(int8_t)(SC1 >> sb);
    const float sc3 = (float)(int)(int8_t)(SC1 >> (16 + sb));
    const float d = half_bits_to_float(r.s4 >> 16);
    float a = sc0 * (S[0] - 32.f * xu.s[0]);
    a += sc1 * (S[1] - 32.f * xu.s[1]);
    a += sc2 * (S[2] - 32.f * xu.s[2]);
    a += sc3 * (S[3] - 32.f * xu.s[3]);
    return d * a;
}

template <> __device__ __forceinline__ void load_raw<Q8_0>(const uint8_t *__restrict__ row, int u, Raw<Q8_0> &r) {
    const uint8_t *B0 = row + u * 36;  // 4-byte aligned
    r.sc = ld_b32(B0);
    r.qa = ld_b128(B0 + 4);
    r.qb = ld_b128(B0 + 20);
}

template <> __device__ __forceinline__ float dot_raw<Q8_0>(const uint8_t *__restrict__, int, const Raw<Q8_0> &r,
                                                           const XUnit<Q8_0> &xu) {
    const uint32_t q[8] = {r.qa.x, r.qa.y, r.qa.z, r.qa.w, r.qb.x, r.qb.y, r.qb.z, r.qb.w};
    float S = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) S = dot4u(q[i] ^ 0x80808080u, xu.v + 4 * i, S);  // q + 128
    return __builtin_bit_cast(float, r.sc) * (S - 128.f * xu.s[0]);
}

__device__ __forceinline__ const uint8_t *q40_window(const uint8_t *row, int u, uint32_t &m) {
    const uint8_t *Q0 = row + u * 18 + 2;  // the block's 16 nibble bytes
    m = (uint32_t)(uintptr_t)Q0 & 3u;      // 2 (even block) or 0 (odd block)
    return Q0 - m;
}

template <> __device__ __forceinline__ void load_raw<Q4_0>(const uint8_t *__restrict__ row, int u, Raw<Q4_0> &r) {
    uint32_t m;
    const uint8_t *A0 = q40_window(row, u, m);
    r.w = ld_b128(A0);
    r.w4 = ld_b32(A0 + 12 + 2 * m);  // bytes 16..19 of the window when m == 2
}

// ---- the ggml-layout formats

// Q5_K: Q4_K's unit (nibble group g: sub-blocks 2g, 2g+1) plus the 32 qh
// bytes, of which the unit uses bits 2g and 2g+1. Codes 0..31 are converted
// one byte per instruction.
template <> __device__ __forceinline__ void load_raw<Q5_K>(const uint8_t *__restrict__ row, int u, Raw<Q5_K> &r) {
    const uint8_t *blk = row + (u >> 2) * 176;  // 176 = 11 * 16: 16-byte aligned
    const int g = u & 3;
    r.h = ld_b128(blk);
    r.ha = ld_b128(blk + 16);
    r.hb = ld_b128(blk + 32);
    r.qa = ld_b128(blk + 48 + 32 * g);
    r.qb = ld_b128(blk + 64 + 32 * g);
}

template <> __device__ __forceinline__ float dot_raw<Q5_K>(const uint8_t *__restrict__, int u, const Raw<Q5_K> &r,
                                                           const XUnit<Q5_K> &xu) {
    const int g = u & 3;
    const uint32_t q[8] = {r.qa.x, r.qa.y, r.qa.z, r.qa.w, r.qb.x, r.qb.y, r.qb.z, r.qb.w};
    const uint32_t H[8] = {r.ha.x, r.ha.y, r.ha.z, r.ha.w, r.hb.x, r.hb.y, r.hb.z, r.hb.w};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const uint32_t hg = H[i] >> (2 * g);  // bit 0 of each byte: sub-block 2g, bit 1: 2g+1
        const uint32_t c0 = (q[i] & 0x0F0F0F0Fu) | ((hg << 4) & 0x10101010u);
        const uint32_t c1 = ((q[i] >> 4) & 0x0F0F0F0Fu) | ((hg << 3) & 0x10101010u);
        s0 = dot4u(c0, xu.v + 4 * i, s0);
        s1 = dot4u(c1, xu.v + 32 + 4 * i, s1);
    }
    const u32x4 h = r.h;
    const uint32_t sc_lo = h.y & 0x3F3F3F3Fu;
    const uint32_t mn_lo = h.z & 0x3F3F3F3Fu;
    const uint32_t sc_hi = (h.w & 0x0F0F0F0Fu) | ((h.y >> 2) & 0x30303030u);
    const uint32_t mn_hi = ((h.w >> 4) & 0x0F0F0F0Fu) | ((h.z >> 2) & 0x30303030u);
    const uint32_t SC = g < 2 ? sc_lo : sc_hi;
    const uint32_t MN = g < 2 ? mn_lo : mn_hi;
    const int sh = 16 * (g & 1);
    const float sc0 = (float)((SC >> sh) & 0xFFu), sc1 = (float)((SC >> (sh + 8)) & 0xFFu);
    const float mn0 = (float)((MN >> sh) & 0xFFu), mn1 = (float)((MN >> (sh + 8)) & 0xFFu);
    const float d = half_bits_to_float(h.x & 0xFFFFu);
    const float dmin = half_bits_to_float(h.x >> 16);
    const float a = sc0 * s0 + sc1 * s1;
    const float m = mn0 * xu.s[0] + mn1 * xu.s[1];
    return d * a - dmin * m;
}

// Q2_K: unit = 16 code bytes (positions l0 .. l0+15 of half h, all four
// quarters: bits 2j, 2j+1 of each byte), the unit's four scale bytes
// (8h + 2j + l0/16) among the 8 of the half, and d|dmin.
template <> __device__ __forceinline__ void load_raw<Q2_K>(const uint8_t *__restrict__ row, int u, Raw<Q2_K> &r) {
    const uint8_t *blk = row + (u >> 2) * 84;  // 84 = 21 * 4: 4-byte aligned
    const int h = (u >> 1) & 1, l0 = 16 * (u & 1);
    r.q = ld_b128(blk + 16 + 32 * h + l0);
    r.s = ld_b64(blk + 8 * h);
    r.dd = ld_b32(blk + 80);
}

template <> __device__ __forceinline__ float dot_raw<Q2_K>(const uint8_t *__restrict__, int u, const Raw<Q2_K> &r,
                                                           const XUnit<Q2_K> &xu) {
    const int p = u & 1;
    const uint32_t Q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
    float S[4] = {0.f, 0.f, 0.f, 0.f};  // scaled by 2^-9
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int j = 0; j < 4; j++) S[j] = dot4_nib((Q[i] >> (2 * j)) & 0x03030303u, xu.v + 16 * j + 4 * i, S[j]);
    }
    float a = 0.f, m = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        // scale byte 2j + p of the half's eight
        const uint32_t sb = ((j < 2 ? r.s.x : r.s.y) >> (8 * (2 * (j & 1) + p))) & 0xFFu;
        a += (float)(sb & 0xFu) * S[j];
        m += (float)(sb >> 4) * xu.s[j];
    }
    const float d = half_bits_to_float(r.dd & 0xFFFFu), dmin = half_bits_to_float(r.dd >> 16);
    return (d * 512.f) * a - dmin * m;
}

// Q3_K: 110-byte blocks are 2-byte aligned; with an even block count per
// row an even block starts 4-byte aligned and an odd one 2 bytes past. Each
// piece is read from the 4-byte boundary at or below it, with one more dword
// for the realignment; the scale window (bytes 96..111 of the even block,
// 94..109 of the odd one) stays inside the block pair.
__device__ __forceinline__ const uint8_t *q3k_block(const uint8_t *row, int u, uint32_t &mis) {
    const uint8_t *B0 = row + (u >> 2) * 110;
    mis = (uint32_t)(uintptr_t)B0 & 3u;
    return B0 - mis;
}

template <> __device__ __forceinline__ void load_raw<Q3_K>(const uint8_t *__restrict__ row, int u, Raw<Q3_K> &r) {
    const int h = (u >> 1) & 1, l0 = 16 * (u & 1);
    uint32_t mis;
    const uint8_t *A0 = q3k_block(row, u, mis);
    r.hm = ld_b128(A0 + l0);  // hmask[l0 .. l0+15]
    r.hm4 = ld_b32(A0 + l0 + 16);
    r.q = ld_b128(A0 + 32 + 32 * h + l0);
    r.q4 = ld_b32(A0 + 48 + 32 * h + l0);
    r.s = ld_b128(A0 + 96);  // packed scales and d
}

template <> __device__ __forceinline__ float dot_raw<Q3_K>(const uint8_t *__restrict__ row, int u, const Raw<Q3_K> &r,
                                                           const XUnit<Q3_K> &xu) {
    const int h = (u >> 1) & 1, p = u & 1;
    uint32_t mis;
    (void)q3k_block(row, u, mis);
    const uint32_t QQ[4] = {align_bytes(r.q.y, r.q.x, mis), align_bytes(r.q.z, r.q.y, mis),
                            align_bytes(r.q.w, r.q.z, mis), align_bytes(r.q4, r.q.w, mis)};
    const uint32_t HM[4] = {align_bytes(r.hm.y, r.hm.x, mis) >> (4 * h), align_bytes(r.hm.z, r.hm.y, mis) >> (4 * h),
                            align_bytes(r.hm.w, r.hm.z, mis) >> (4 * h), align_bytes(r.hm4, r.hm.w, mis) >> (4 * h)};
    float S[4] = {0.f, 0.f, 0.f, 0.f};  // sums of (q + 4) x, scaled by 2^-9
#pragma unroll
    for (int i = 0; i < 4; i++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            // code + 4 = low 2 bits | hmask bit j (of this half) << 2, in 0..7
            const uint32_t hb = j <= 2 ? (HM[i] << (2 - j)) : (HM[i] >> (j - 2));
            const uint32_t c = ((QQ[i] >> (2 * j)) & 0x03030303u) | (hb & 0x04040404u);
            S[j] = dot4_nib(c, xu.v + 16 * j + 4 * i, S[j]);
        }
    }
    const uint32_t SC0 = align_bytes(r.s.y, r.s.x, mis), SC1 = align_bytes(r.s.z, r.s.y, mis);
    const uint32_t SC2 = align_bytes(r.s.w, r.s.z, mis);
    float a = 0.f;
#pragma unroll
    for (int j = 0; j < 4; j++) {
        // scale 8h + 2j + p: low 4 bits in packed byte 2j + p (low nibble in
        // half 0, high nibble in half 1), top 2 bits at bit 2(2h + j/2) of
        // packed byte 8 + 2(j&1) + p
        const int bi = 2 * (j & 1) + p;
        const uint32_t lo4 = ((j < 2 ? SC0 : SC1) >> (8 * bi + 4 * h)) & 0xFu;
        const uint32_t hi2 = (SC2 >> (8 * bi + 2 * (2 * h + (j >> 1)))) & 3u;
        const float sc = (float)((int)(lo4 | (hi2 << 4)) - 32);
        a += sc * (512.f * S[j] - 4.f * xu.s[j]);
    }
    const float d = half_bits_to_float((r.s.w >> (8 * mis)) & 0xFFFFu);
    return d * a;
}

// Q5_1: one 24-byte block (8-byte aligned) per unit: d|m, qh, 16 nibble
// bytes. The fifth bits are spread to bit 4 of each code byte.
template <> __device__ __forceinline__ void load_raw<Q5_1>(const uint8_t *__restrict__ row, int u, Raw<Q5_1> &r) {
    const uint8_t *blk = row + u * 24;
    r.h = ld_b64(blk);
    r.q = ld_b128(blk + 8);
}

// bits 0..3 of n -> bit 4 of bytes 0..3
__device__ __forceinline__ uint32_t spread4_to_bit4(uint32_t n) { return ((n & 0xFu) * 0x00204081u << 4) & 0x10101010u; }

template <> __device__ __forceinline__ float dot_raw<Q5_1>(const uint8_t *__restrict__, int, const Raw<Q5_1> &r,
                                                           const XUnit<Q5_1> &xu) {
    const uint32_t qh = r.h.y;
    const uint32_t q[4] = {r.q.x, r.q.y, r.q.z, r.q.w};
    float S = 0.f;
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t c0 = (q[i] & 0x0F0F0F0Fu) | spread4_to_bit4(qh >> (4 * i));
        const uint32_t c1 = ((q[i] >> 4) & 0x0F0F0F0Fu) | spread4_to_bit4(qh >> (16 + 4 * i));
        S = dot4u(c0, xu.v + 4 * i, S);
        S = dot4u(c1, xu.v + 16 + 4 * i, S);
    }
    const float d = half_bits_to_float(r.h.x & 0xFFFFu), m = half_bits_to_float(r.h.x >> 16);
    return d * S + m * xu.s[0];
}

// Q8_0_F16: 34-byte blocks, 2-byte aligned; with an even block count per row
// an even block starts 4-byte aligned. The 32 codes are read from the 4-byte
// boundary at or below them (9 dwords for an even block, 8 for an odd one,
// whose ninth load re-reads an in-block dword) and realigned; an odd block's
// scale is the top half of the even block's ninth dword (the lane below,
// same 16-lane DPP row).
__device__ __forceinline__ const uint8_t *q80h_window(const uint8_t *row, int u, uint32_t &s) {
    const uint8_t *Q = row + u * 34 + 2;  // the block's codes
    s = (uint32_t)(uintptr_t)Q & 3u;      // 2 (even block) or 0 (odd block)
    return Q - s;
}

template <> __device__ __forceinline__ void load_raw<Q8_0_F16>(const uint8_t *__restrict__ row, int u,
                                                               Raw<Q8_0_F16> &r) {
    uint32_t s;
    const uint8_t *A0 = q80h_window(row, u, s);
    r.a = ld_b128(A0);
    r.b = ld_b128(A0 + 16);
    r.c = ld_b32(A0 + 28 + 2 * s);  // bytes 32..35 of the window when s == 2
}

template <> __device__ __forceinline__ float dot_raw<Q8_0_F16>(const uint8_t *__restrict__ row, int u,
                                                               const Raw<Q8_0_F16> &r, const XUnit<Q8_0_F16> &xu) {
    uint32_t s;
    (void)q80h_window(row, u, s);
    const uint32_t w[9] = {r.a.x, r.a.y, r.a.z, r.a.w, r.b.x, r.b.y, r.b.z, r.b.w, r.c};
    float S = 0.f;
#pragma unroll
    for (int k = 0; k < 8; k++) S = dot4u(align_bytes(w[k + 1], w[k], s) ^ 0x80808080u, xu.v + 4 * k, S);  // q + 128
    const uint32_t prev_c = dpp_mov<DPP_SHR1>(r.c);
    const uint32_t dbits = s ? (r.a.x & 0xFFFFu) : (prev_c >> 16);
    return half_bits_to_float(dbits) * (S - 128.f * xu.s[0]);
}

// The same pieces read from a copy of the row in LDS (streamed mode). The
// copy keeps the row's alignment modulo 16, so Q4_K pieces are 16-byte
// aligned there and the realignment of the others is unchanged.
template <int F> __device__ __forceinline__ void lds_raw(const uint8_t *row, int u, Raw<F> &r) { load_raw<F>(row, u, r); }
template <> __device__ __forceinline__ void lds_raw<Q4_K>(const uint8_t *row, int u, Raw<Q4_K> &r) {
    const uint8_t *blk = static_cast<const uint8_t *>(__builtin_assume_aligned(row + (u >> 2) * 144, 16));
    const int g = u & 3;
    r.h = *reinterpret_cast<const u32x4 *>(blk);
    r.qa = *reinterpret_cast<const u32x4 *>(blk + 16 + 32 * g);
    r.qb = *reinterpret_cast<const u32x4 *>(blk + 32 + 32 * g);
}

// Q6_K windows are only 4-byte aligned: read them from LDS as dword pairs
// (ds_read2_b32), which need no more than 4-byte alignment.
__device__ __forceinline__ u32x4 lds_b128_a4(const uint8_t *p) {
    const uint32_t *q = static_cast<const uint32_t *>(__builtin_assume_aligned(p, 4));
    uint32_t a = q[0], b = q[1], c = q[2], d = q[3];
    __asm__("" : "+v"(a), "+v"(b));
    return u32x4{a, b, c, d};
}
__device__ __forceinline__ uint32_t lds_b32(const uint8_t *p) {
    return *static_cast<const uint32_t *>(__builtin_assume_aligned(p, 4));
}
template <> __device__ __forceinline__ void lds_raw<Q6_K>(const uint8_t *row, int u, Raw<Q6_K> &r) {
    const int h = (u >> 1) & 1, l0 = 16 * (u & 1);
    uint32_t mis;
    const uint8_t *A0 = q6k_block(row, u, mis);
    r.p[0] = lds_b128_a4(A0 + 64 * h + l0);
    r.p[1] = lds_b128_a4(A0 + 64 * h + 32 + l0);
    r.p[2] = lds_b128_a4(A0 + 128 + 32 * h + l0);
    r.s = lds_b128_a4(A0 + 192);
    const uint16_t *t = static_cast<const uint16_t *>(__builtin_assume_aligned(A0 + mis + 206, 2));
    r.s4 = (uint32_t)t[0] | ((uint32_t)t[1] << 16);
    r.e[0] = lds_b32(A0 + 64 * h + l0 + 16);
    r.e[1] = lds_b32(A0 + 64 * h + 32 + l0 + 16);
    r.e[2] = lds_b32(A0 + 128 + 32 * h + l0 + 16);
}

// The ggml-layout formats in LDS: Q5_K pieces are 16-byte aligned (blocks of
// 11 * 16 bytes); Q5_1 pieces 8-byte aligned (read as 8-byte pairs); the
// Q2_K, Q3_K and Q8_0_F16 windows 4-byte aligned (read as dword pairs).
__device__ __forceinline__ u32x4 lds_b128_a8(const uint8_t *p) {
    const uint64_t *q = static_cast<const uint64_t *>(__builtin_assume_aligned(p, 8));
    uint64_t a = q[0], b = q[1];
    __asm__("" : "+v"(a));
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32), (uint32_t)b, (uint32_t)(b >> 32)};
}
template <> __device__ __forceinline__ void lds_raw<Q5_K>(const uint8_t *row, int u, Raw<Q5_K> &r) {
    const uint8_t *blk = static_cast<const uint8_t *>(__builtin_assume_aligned(row + (u >> 2) * 176, 16));
    const int g = u & 3;
    r.h = *reinterpret_cast<const u32x4 *>(blk);
    r.ha = *reinterpret_cast<const u32x4 *>(blk + 16);
    r.hb = *reinterpret_cast<const u32x4 *>(blk + 32);
    r.qa = *reinterpret_cast<const u32x4 *>(blk + 48 + 32 * g);
    r.qb = *reinterpret_cast<const u32x4 *>(blk + 64 + 32 * g);
}
template <> __device__ __forceinline__ void lds_raw<Q5_1>(const uint8_t *row, int u, Raw<Q5_1> &r) {
    const uint8_t *blk = row + u * 24;
    const uint64_t h = *static_cast<const uint64_t *>(__builtin_assume_aligned(blk, 8));
    r.h = u32x2{(uint32_t)h, (uint32_t)(h >> 32)};
    r.q = lds_b128_a8(blk + 8);
}
template <> __device__ __forceinline__ void lds_raw<Q2_K>(const uint8_t *row, int u, Raw<Q2_K> &r) {
    const uint8_t *blk = row + (u >> 2) * 84;
    const int h = (u >> 1) & 1, l0 = 16 * (u & 1);
    r.q = lds_b128_a4(blk + 16 + 32 * h + l0);
    r.s = u32x2{lds_b32(blk + 8 * h), lds_b32(blk + 8 * h + 4)};
    r.dd = lds_b32(blk + 80);
}
template <> __device__ __forceinline__ void lds_raw<Q3_K>(const uint8_t *row, int u, Raw<Q3_K> &r) {
    const int h = (u >> 1) & 1, l0 = 16 * (u & 1);
    uint32_t mis;
    const uint8_t *A0 = q3k_block(row, u, mis);
    r.hm = lds_b128_a4(A0 + l0);
    r.hm4 = lds_b32(A0 + l0 + 16);
    r.q = lds_b128_a4(A0 + 32 + 32 * h + l0);
    r.q4 = lds_b32(A0 + 48 + 32 * h + l0);
    r.s = lds_b128_a4(A0 + 96);
}
template <> __device__ __forceinline__ void lds_raw<Q8_0_F16>(const uint8_t *row, int u, Raw<Q8_0_F16> &r) {
    uint32_t s;
    const uint8_t *A0 = q80h_window(row, u, s);
    r.a = lds_b128_a4(A0);
    r.b = lds_b128_a4(A0 + 16);
    r.c = lds_b32(A0 + 28 + 2 * s);
}

template <> __device__ __forceinline__ float dot_raw<Q4_0>(const uint8_t *__restrict__ row, int u, const Raw<Q4_0> &r,
                                                           const XUnit<Q4_0> &xu) {
    uint32_t m;
    (void)q40_window(row, u, m);
    const u32x4 w = r.w;
    const uint32_t q[4] = {align_bytes(w.y, w.x, m), align_bytes(w.z, w.y, m), align_bytes(w.w, w.z, m),
                           align_bytes(r.w4, w.w, m)};
    // The scale: an even block (m == 2) starts at its window, so d is the
    // window's first two bytes; an odd block's d is the last two bytes that
    // the even block before it (the lane below, same 16-lane DPP row) read
    // past its own nibbles.
    const uint32_t prev_w4 = dpp_mov<DPP_SHR1>(r.w4);
    const uint32_t dbits = m ? (w.x & 0xFFFFu) : (prev_w4 >> 16);
    float S = 0.f;  // scaled by 2^-9
#pragma unroll
    for (int i = 0; i < 4; i++) {
        S = dot4_nib(q[i] & 0x0F0F0F0Fu, xu.v + 4 * i, S);             // weights 4i..4i+3
        S = dot4_nib((q[i] >> 4) & 0x0F0F0F0Fu, xu.v + 16 + 4 * i, S);  // weights 16+4i..
    }
    return half_bits_to_float(dbits) * (512.f * S - 8.f * xu.s[0]);
}

// v + (v from the lane selected by a DPP control), lane-wise.
template <int CTRL> __device__ __forceinline__ float dpp_add(float v) {
    const int o = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false);
    return v + __builtin_bit_cast(float, o);
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Sum of v over the lanes of each aligned group of min(2^Lshift, 16) lanes;
// every lane of the group gets the sum. DPP: quad_perm [1,0,3,2] and
// [2,3,0,1], then row_half_mirror (8 lanes) and row_mirror (16 lanes).
__device__ __forceinline__ float reduce16(float v, int Lshift) {
    if (Lshift >= 1) v = dpp_add<0xB1>(v);
    if (Lshift >= 2) v = dpp_add<0x4E>(v);
    if (Lshift >= 3) v = dpp_add<0x141>(v);
    if (Lshift >= 4) v = dpp_add<0x140>(v);
    return v;
}

// Up to kMaxMats weight matrices of the same width, read against the same x,
// in one launch. Matrices 0..n1-1 have the launch's first format and the
// rest its second (the two formats of a launch share one GemvPlan). Matrix j
// starts wof[j] bytes after W and writes y + yof[j]. Each matrix has its own
// range of workgroups, starting at wgbeg[j]; workgroup b of matrix j (counted
// from wgbeg[j]) owns q[j] + (b < r[j]) consecutive row groups of NWR * RP
// rows, so no workgroup divides to find its rows.
constexpr int kMaxMats = kGemvMaxMats;
struct GemvWork {
    const float *x;
    const uint8_t *W;
    float *y;
    GemvInput in;  // the transform of x (kind 0: none)
    int64_t wof[kMaxMats];
    int64_t yof[kMaxMats];
    int rows[kMaxMats];
    int wgbeg[kMaxMats];  // entries past the last matrix hold the grid size
    int q[kMaxMats], r[kMaxMats];
    int n1;
    int row_bytes[2];  // per format
};

// What one workgroup needs from the kernel arguments: its matrix and rows,
// and the lane plan.
struct MatSel {
    const uint8_t *W;
    float *y;
    int rows;
    int g0, g1;  // row groups [g0, g1) of the matrix
    int j;       // matrix index
    int row_bytes;
    GemvPlan p;
};

// Every scalar is read in one round of scalar loads at the top of the kernel:
// the empty asm statements, placed together, make all of them values before
// any other work, so the choice among table entries is a select of
// registers (a select of argument addresses would cost a second round).
static_assert(kMaxMats == 4, "mat_sel is written out for four matrices");
__device__ __forceinline__ MatSel mat_sel(const GemvWork &w, const GemvPlan &pa, int blk) {
    int64_t o1 = w.wof[1], o2 = w.wof[2], o3 = w.wof[3], p1 = w.yof[1], p2 = w.yof[2], p3 = w.yof[3];
    int r0 = w.rows[0], r1 = w.rows[1], r2 = w.rows[2], r3 = w.rows[3];
    int b1 = w.wgbeg[1], b2 = w.wgbeg[2], b3 = w.wgbeg[3];
    int q0 = w.q[0], q1 = w.q[1], q2 = w.q[2], q3 = w.q[3];
    int e0 = w.r[0], e1 = w.r[1], e2 = w.r[2], e3 = w.r[3];
    int n1 = w.n1, rb0 = w.row_bytes[0], rb1 = w.row_bytes[1];
    GemvPlan p = pa;
    __asm__("" : "+s"(o1), "+s"(o2), "+s"(o3), "+s"(p1), "+s"(p2), "+s"(p3));
    __asm__("" : "+s"(r0), "+s"(r1), "+s"(r2), "+s"(r3), "+s"(b1), "+s"(b2), "+s"(b3), "+s"(n1), "+s"(rb0),
            "+s"(rb1));
    __asm__("" : "+s"(q0), "+s"(q1), "+s"(q2), "+s"(q3), "+s"(e0), "+s"(e1), "+s"(e2), "+s"(e3));
    __asm__("" : "+s"(p.U), "+s"(p.KS), "+s"(p.Uw), "+s"(p.Lshift), "+s"(p.RP), "+s"(p.NWR), "+s"(p.ksmul));
    const int j = (blk >= b1) + (blk >= b2) + (blk >= b3);
    const int b = blk - (j == 0 ? 0 : j == 1 ? b1 : j == 2 ? b2 : b3);
    const int q = j == 0 ? q0 : j == 1 ? q1 : j == 2 ? q2 : q3;
    const int r = j == 0 ? e0 : j == 1 ? e1 : j == 2 ? e2 : e3;
    MatSel s;
    s.W = w.W + (j == 0 ? 0 : j == 1 ? o1 : j == 2 ? o2 : o3);
    s.y = w.y + (j == 0 ? 0 : j == 1 ? p1 : j == 2 ? p2 : p3);
    s.rows = j == 0 ? r0 : j == 1 ? r1 : j == 2 ? r2 : r3;
    s.g0 = b * q + min(b, r);
    s.g1 = s.g0 + q + (b < r ? 1 : 0);
    s.j = j < n1 ? 0 : 1;  // format segment
    s.row_bytes = j < n1 ? rb0 : rb1;
    s.p = p;
    return s;
}

// DEPTH row buffers rotate: while one row is decoded, the loads of the next
// DEPTH-1 rows of this lane are in flight. Loads are unconditional (a row past
// the end of its matrix is clamped to the last row, a real row whose value is
// then written twice) and the main loop holds no global stores, barriers or
// other memory writes that count against the load counter, so the wait
// before each decode covers only that row's buffer. After the main loop the
// last (fewer than DEPTH) groups are already in the buffers and are decoded
// without further loads. With a row's units split over KS waves, the KS
// partial sums go to LDS and are added at the end in a fixed order.
//
// Streamed mode (SPL > 0): the rows of one row group are consecutive, so the
// group is one contiguous byte range. All threads of the workgroup read it
// as consecutive 16-byte pieces (each load instruction covers whole cache
// lines, SPL pieces per thread) with the streaming cache policy, and write
// it to one of two LDS slots; each lane then reads its unit from LDS exactly
// as it would from HBM. The loads of the next DEPTH groups are in flight
// while a group is decoded, one barrier per group.
//
// XF transforms x as it is staged (the work that feeds a projection in a
// decode step, done by the projection itself): XF = 1, x' = RMSNorm(x + aux)
// * norm_w, with the sum of squares taken by each workgroup over the whole
// of x + aux (every workgroup stages all of x anyway), and workgroup 0
// writing x + aux to x_out at its end (the residual stream; x_out is not x,
// which other workgroups may still be reading); XF = 2, x' = silu(x) * aux.
// The norm's factor 1/rms is one scalar and the product is linear in x, so
// XF = 1 stages norm_w * (x + aux) at once and multiplies each row's sum by
// the factor: the sum of squares is reduced across the workgroup behind the
// barrier that x's staging needs anyway, not on the way to it.
//
// XLOOP (rows wider than the register staging holds): x is staged in rounds
// of one 16-byte chunk per thread, after the first weight loads are issued
// (their latency then covers the staging).
template <int F, int DEPTH, bool SPLIT, bool WIDE, int SPL, int XF = 0, bool XLOOP = false>
__device__ __forceinline__ void gemv_body(const float *__restrict__ x, const MatSel &ms, float *res,
                                          const GemvInput &xin) {
    // Everything up to the first loads depends only on the kernel arguments
    // (one round of scalar loads) and the thread id.
    const GemvPlan &p = ms.p;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nthreads = 64 * p.KS * p.NWR;
    const int wr = (wave * p.ksmul) >> 16;
    const int ks = wave - wr * p.KS;
    const int slot = lane >> p.Lshift, li = lane & ((1 << p.Lshift) - 1);
    const int u_raw = ks * p.Uw + li;
    const bool active = li < p.Uw && u_raw < p.U;
    const int u = active ? u_raw : 0;  // idle lanes read unit 0 and drop it
    const int RG = p.NWR * p.RP;
    const int g0 = ms.g0, g1 = ms.g1;
    const int row_bytes = ms.row_bytes;
    const int nloc = (g1 - g0) * RG;  // rows of this workgroup
    const int rofs = wr * p.RP + slot;
    const int64_t lane_ofs = (int64_t)rofs * row_bytes;
    const int64_t gstride = (int64_t)RG * row_bytes;
    const uint8_t *const Wm = ms.W;
    const int rows = ms.rows;
    const uint8_t *const last_row = Wm + (int64_t)(rows - 1) * row_bytes;
    // Packed bytes of this lane's row in group g (g clamped to this
    // workgroup's groups, the row to the matrix).
    auto row_ptr = [&](int g) {
        const int gg = min(g, g1 - 1);
        return gg * RG + rofs < rows ? Wm + gg * gstride + lane_ofs : last_row;
    };

    // LDS: [x, padded][sums of x per 16 floats][KS partial results]. In the
    // streamed mode the two group slots (16-byte aligned) reuse the space of
    // x once every lane holds its x in registers, and the partial results
    // follow the larger of the two.
    const int cols = p.U * Unit<F>::W;
    float *xs = res;
    float *xsum = res + xpos(cols);
    const int x_fl = (xpos(cols) + (cols >> 4) + 3) & ~3;  // floats of x and its sums, rounded to 16 bytes
    // streamed mode: pieces per group slot (the group from the 128-byte
    // boundary at or below its first byte, so that every load instruction
    // covers whole cache lines, to at least 4 bytes past its last), and the
    // last whole piece of the matrix (its size is a multiple of 16 bytes)
    const int NP = SPL > 0 ? (int)((gstride + 159) >> 4) : 0;
    const int64_t T16 = (int64_t)rows * row_bytes - 16;
    uint8_t *const slots = reinterpret_cast<uint8_t *>(res);
    float *const part0 = SPL > 0 ? res + max(x_fl, 8 * NP) : xsum + (cols >> 4);
    float *mine = part0 + ks * nloc;

    // x: coalesced 16-byte loads by all threads, issued first; then the
    // first rows' weights, so that their latency overlaps the staging of x.
    // Scheduling barriers keep each group of loads together and in order:
    // the load counter is in-order, so a wait for one group covers only the
    // loads issued before it.
    // (the host keeps cols <= 32 * threads unless XLOOP)
    constexpr int XCH = XLOOP ? 1 : 8;  // 16-byte chunks of x per thread
    constexpr int XA = XF != 0 ? XCH : 1, XW = XF == 1 ? XCH : 1;
    float4 xv[XCH], av[XA], wv[XW];
    if constexpr (!XLOOP) {
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            const int c = threadIdx.x + i * nthreads;
            const bool in = 4 * c < cols;
            xv[i] = in ? *reinterpret_cast<const float4 *>(x + 4 * c) : float4{0.f, 0.f, 0.f, 0.f};
            if constexpr (XF != 0)
                av[i] = in ? *reinterpret_cast<const float4 *>(xin.aux + 4 * c) : float4{0.f, 0.f, 0.f, 0.f};
            if constexpr (XF == 1)
                wv[i] = in ? *reinterpret_cast<const float4 *>(xin.norm_w + 4 * c) : float4{0.f, 0.f, 0.f, 0.f};
        }
    }
    __builtin_amdgcn_sched_barrier(0);

    // streamed mode: the first byte (rounded down to 128) of group g, the
    // pieces of group g into a stream buffer and from it into slot s. Thread
    // t takes pieces t, t + nthreads, ... of the group, clamped to its last
    // piece and to the last piece of the matrix (all limits are uniform, so
    // a piece costs one min per load and per store). The loads of a group
    // past this workgroup's last one read x instead (from L2; what they
    // bring is never decoded), so no weight byte is read twice.
    auto gbase = [&](int g) { return ((int64_t)g * gstride) & ~(int64_t)127; };
    const uint8_t *const xb = reinterpret_cast<const uint8_t *>(x);
    auto src_of = [&](int g, uint32_t &lim) {  // base address and last piece offset of group g
        const bool in = g < g1;
        const int64_t b = gbase(g);
        const int64_t last = in ? min((int64_t)16 * (NP - 1), T16 - b) : (int64_t)min(16 * (NP - 1), 4 * cols - 16);
        lim = (uint32_t)last;
        return in ? Wm + b : xb;
    };
    auto sload = [&](int g, u32x4 *sb) {
        uint32_t lim;
        const uint8_t *src = src_of(g, lim);
#pragma unroll
        for (int k = 0; k < SPL; k++) {
            const uint32_t o = min((uint32_t)(16 * (threadIdx.x + k * nthreads)), lim);
            sb[k] = ld_b128_nt(src + o);
        }
    };
    auto sstore = [&](int g, int s, const u32x4 *sb) {
        uint32_t lim;
        (void)src_of(g, lim);
        uint8_t *dst = slots + s * 16 * NP;
#pragma unroll
        for (int k = 0; k < SPL; k++) {
            const uint32_t o = min((uint32_t)(16 * (threadIdx.x + k * nthreads)), lim);
            *reinterpret_cast<u32x4 *>(dst + o) = sb[k];
        }
    };
    auto lrow = [&](int g, int s) {  // this lane's row of group g (< g1) in slot s
        const int r = min(g * RG + rofs, rows - 1);
        return static_cast<const uint8_t *>(slots + s * 16 * NP + ((int64_t)r * row_bytes - gbase(g)));
    };

    constexpr int NB = SPL > 0 ? DEPTH : DEPTH - 1;  // buffers loaded before the loop
    Raw<F> buf[DEPTH];
    u32x4 sbuf[DEPTH][SPL > 0 ? SPL : 1];
#pragma unroll
    for (int d = 0; d < NB; d++) {
        if constexpr (SPL > 0)
            sload(g0 + d, sbuf[d]);
        else
            load_raw<F>(row_ptr(g0 + d), u, buf[d]);
        __builtin_amdgcn_sched_barrier(0);
    }
    // chunk c of x' (4 floats, thread c % nthreads) into LDS, and the sum of
    // its aligned group of 16 floats: 4 consecutive chunks = 4 lanes
    auto put_x = [&](int c, const float4 &v) {
        float t = (v.x + v.y) + (v.z + v.w);
        t = dpp_add<0xB1>(t);
        t = dpp_add<0x4E>(t);
        if (4 * c < cols) {
            *reinterpret_cast<float4 *>(xs + xpos(4 * c)) = v;
            if ((c & 3) == 0) xsum[c >> 2] = t;
        }
    };
    // __expf (v_exp_f32 on g * log2 e) and the hardware reciprocal (v_rcp_f32,
    // 1 ulp) instead of expf and an IEEE division: a few ulps, far inside the
    // GEMV's tolerance, at a fraction of the cost; every workgroup evaluates
    // it over all of x. (Large negative g: the reciprocal of inf is 0.)
    auto silu_mul = [](float g, float u) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u; };
    // each wave's part of sum(t^2) into red (read after the staging's
    // barrier by inv_rms: 1 / sqrt(mean(t^2) + eps), the same order of
    // additions in every thread)
    __shared__ float red[8];
    auto put_ss = [&](float ss) {
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        if (lane == 0) red[wave] = ss;
    };
    auto inv_rms = [&]() {
        float tot = 0.f;
        for (int i = 0; i < nthreads / 64; i++) tot += red[i];
        return 1.0f / sqrtf(tot / (float)cols + xin.eps);
    };
    if constexpr (XLOOP) {
        // batches of XB chunks per thread (uniform trip count), each batch's
        // loads issued before its first store
        constexpr int XB = 8;
        float ss = 0.f;
        for (int c0 = 0; 4 * c0 < cols; c0 += XB * nthreads) {
            float4 v[XB], a[XF != 0 ? XB : 1], g[XF == 1 ? XB : 1];
#pragma unroll
            for (int i = 0; i < XB; i++) {
                const int c = c0 + threadIdx.x + i * nthreads;
                const bool in = 4 * c < cols;
                v[i] = in ? *reinterpret_cast<const float4 *>(x + 4 * c) : float4{0.f, 0.f, 0.f, 0.f};
                if constexpr (XF != 0)
                    a[i] = in ? *reinterpret_cast<const float4 *>(xin.aux + 4 * c) : float4{0.f, 0.f, 0.f, 0.f};
                if constexpr (XF == 1)
                    g[i] = in ? *reinterpret_cast<const float4 *>(xin.norm_w + 4 * c) : float4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
            for (int i = 0; i < XB; i++) {
                const int c = c0 + threadIdx.x + i * nthreads;
                if constexpr (XF == 1) {
                    const float4 t = float4{v[i].x + a[i].x, v[i].y + a[i].y, v[i].z + a[i].z, v[i].w + a[i].w};
                    ss += t.x * t.x + t.y * t.y + t.z * t.z + t.w * t.w;
                    v[i] = float4{g[i].x * t.x, g[i].y * t.y, g[i].z * t.z, g[i].w * t.w};
                } else if constexpr (XF == 2) {
                    v[i] = float4{silu_mul(v[i].x, a[i].x), silu_mul(v[i].y, a[i].y), silu_mul(v[i].z, a[i].z),
                                  silu_mul(v[i].w, a[i].w)};
                }
                put_x(c, v[i]);
            }
        }
        if constexpr (XF == 1) put_ss(ss);
    } else if constexpr (XF == 1) {
        // t = x + aux; staged: norm_w * t (the factor 1 / sqrt(mean(t^2) + eps)
        // multiplies each row's sum)
        float ss = 0.f;
#pragma unroll
        for (int i = 0; i < XCH; i++) {
            xv[i] = float4{xv[i].x + av[i].x, xv[i].y + av[i].y, xv[i].z + av[i].z, xv[i].w + av[i].w};
            ss += xv[i].x * xv[i].x + xv[i].y * xv[i].y + xv[i].z * xv[i].z + xv[i].w * xv[i].w;
        }
        put_ss(ss);
#pragma unroll
        for (int i = 0; i < XCH; i++)
            xv[i] = float4{wv[i].x * xv[i].x, wv[i].y * xv[i].y, wv[i].z * xv[i].z, wv[i].w * xv[i].w};
    } else if constexpr (XF == 2) {
#pragma unroll
        for (int i = 0; i < XCH; i++)
            xv[i] = float4{silu_mul(xv[i].x, av[i].x), silu_mul(xv[i].y, av[i].y), silu_mul(xv[i].z, av[i].z),
                           silu_mul(xv[i].w, av[i].w)};
    }
    if constexpr (!XLOOP) {
#pragma unroll
        for (int i = 0; i < XCH; i++) put_x(threadIdx.x + i * nthreads, xv[i]);
    }
    __syncthreads();
    const float xscale = XF == 1 ? inv_rms() : 1.0f;  // the norm's factor (XF = 1)
    XUnit<F> xu;
    read_x<F>(xs, xsum, u, xu);
    if constexpr (SPL > 0) {
        // the first group goes to slot 0, over x
        __syncthreads();
        sstore(g0, 0, sbuf[0]);
        __syncthreads();
    }
    if (!active) {
#pragma unroll
        for (int i = 0; i < Unit<F>::W; i++) xu.v[i] = 0.f;
#pragma unroll
        for (int i = 0; i < Unit<F>::NSUM; i++) xu.s[i] = 0.f;
    }

    // decode the row of group g (its bytes at row, their raw pieces in bf)
    // and write its result
    auto finish = [&](int g, const uint8_t *row, const Raw<F> &bf) {
        float part = dot_raw<F>(row, u, bf, xu);
        if constexpr (XF == 1) part *= xscale;
        if constexpr (WIDE) {
            // Row slots of 16, 32 or 64 lanes: the full 16-lane butterfly,
            // then the four 16-lane sums combined per slot, all without
            // branches (the slot width only picks among the results).
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
            part = reduce16(part, p.Lshift);  // row slots of at most 8 lanes
        }
        // Every lane of a row slot now holds the row's sum.
        if constexpr (!SPLIT) {
            // All lanes store the same value to the same (clamped) row: no
            // divergent branch around the store, so the load counter waits
            // stay exact.
            ms.y[min(g * RG + rofs, rows - 1)] = part;
        } else if (li == 0) {
            mine[(g - g0) * RG + rofs] = part;
        }
    };

    if constexpr (SPL > 0) {
        // group gc sits in slot (gc - g0) & 1; its stream buffer is refilled
        // with group gc + DEPTH before it is decoded, and group gc + 1 is
        // moved to the other slot after it
        auto step = [&](int gc, u32x4 *mine_sb, const u32x4 *next_sb) {
            sload(gc + DEPTH, mine_sb);
            __builtin_amdgcn_sched_barrier(0);
            const int s = (gc - g0) & 1;
            const uint8_t *row = lrow(gc, s);
            Raw<F> r;
            lds_raw<F>(row, u, r);
            finish(gc, row, r);
            __builtin_amdgcn_sched_barrier(0);  // the wait for group gc + 1 comes after the decode of gc
            sstore(gc + 1, s ^ 1, next_sb);
            __syncthreads();
        };
        int g = g0;
        for (; g + DEPTH <= g1; g += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; d++) step(g + d, sbuf[d], sbuf[(d + 1) % DEPTH]);
        }
#pragma unroll
        for (int d = 0; d < DEPTH - 1; d++)
            if (g + d < g1) step(g + d, sbuf[d], sbuf[(d + 1) % DEPTH]);
    } else {
        int g = g0;
        for (; g + DEPTH <= g1; g += DEPTH) {
#pragma unroll
            for (int d = 0; d < DEPTH; d++) {
                load_raw<F>(row_ptr(g + d + DEPTH - 1), u, buf[(d + DEPTH - 1) % DEPTH]);
                __builtin_amdgcn_sched_barrier(0);
                finish(g + d, row_ptr(g + d), buf[d]);
            }
        }
        // groups g .. g1-1 (fewer than DEPTH) sit in buf[0 ..]
#pragma unroll
        for (int d = 0; d < DEPTH - 1; d++)
            if (g + d < g1) finish(g + d, row_ptr(g + d), buf[d]);
    }

    if constexpr (SPLIT) {
        __syncthreads();
        for (int i = threadIdx.x; i < nloc; i += nthreads) {
            float sum = part0[i];
            for (int k = 1; k < p.KS; k++) sum += part0[k * nloc + i];
            const int r = g0 * RG + i;
            if (r < rows) ms.y[r] = sum;
        }
    }
    if constexpr (XF == 1) {
        // the residual stream: x + aux, written once (by workgroup 0), after
        // its main loop so that no store enters the loop's load waits
        if (blockIdx.x == 0 && xin.x_out) {
            for (int c = threadIdx.x; 4 * c < cols; c += nthreads) {
                const float4 a = *reinterpret_cast<const float4 *>(x + 4 * c);
                const float4 b = *reinterpret_cast<const float4 *>(xin.aux + 4 * c);
                *reinterpret_cast<float4 *>(xin.x_out + 4 * c) = float4{a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w};
            }
        }
    }
}

// ---- plans (host side)

// Floats of LDS for x staged at width cols: x padded (xpos) and the sums
// of x per 16, rounded to 16 bytes.
inline int64_t x_lds_floats(int64_t cols) { return (cols + 4 * (cols / 64) + cols / 16 + 3) & ~(int64_t)3; }
constexpr int64_t kMaxRes = 2048;  // floats of LDS for row results (rows split over waves)

// Rows up to this width stage x from registers (8 chunks of 16 bytes per
// thread); wider rows use the wide-row kernel.
constexpr int64_t kRegStageCols = 6144;

// Whether the fused kernel handles this format and shape (else the generic
// kernel runs): at most 512 units per row, x and the row results fit one
// workgroup's LDS, row and group indices that fit in 32 bits, and for the
// 2-byte aligned formats:
//   q4_0, Q8_0_F16: an even number of blocks per row (every row starts
//     4-byte aligned: an odd block takes its scale from the lane below);
//   Q3_K: each block is read through 4-byte windows from the boundary at or
//     below it, and the scale window ends 2 bytes past a block that starts
//     4-byte aligned; that is harmless except at the last block of the
//     matrix, so rows * blocks per row must be even (the last block then
//     starts 2 bytes past a boundary). (Q6_K reads its last four bytes as
//     two 2-byte loads and has no such rule.)
template <int F> inline bool fast_ok(int64_t rows, int64_t cols) {
    const int64_t nb = cols / Layout<F>::QK;
    const bool pairs = (F == Q4_0 || F == Q8_0_F16);
    const bool windows = (F == Q3_K);
    if (cols / Unit<F>::W > 512 || rows > (int64_t(1) << 30)) return false;
    if ((pairs && nb % 2 != 0) || (windows && nb % 2 != 0 && rows % 2 != 0)) return false;
    // (256 bytes left for the kernels' static LDS: the norm's reduction array)
    return cols <= kRegStageCols || (x_lds_floats(cols) + kMaxRes) * 4 + 256 <= device_lds_per_block();
}

// How the lanes of a workgroup cover rows of width cols (units per row, waves
// per row, lanes per row slot, row waves).
template <int F> inline GemvPlan make_plan(int64_t cols) {
    const int64_t U = cols / Unit<F>::W;
    const int ksmax = cols > kRegStageCols ? 8 : 4;  // waves per row (8 only in the wide-row kernel)
    GemvPlan p;
    p.U = (int)U;
    if (U <= 64) {
        int L = 1, sh = 0;
        while (L < U) {
            L <<= 1;
            sh++;
        }
        p.KS = 1;
        p.Uw = (int)U;
        p.Lshift = sh;
        p.RP = 64 / L;
    } else {
        // Split a row's units over KS waves, each wave covering Uw units of
        // one row (64 lanes) or of each of two rows (32 lanes per row),
        // whichever leaves fewer lanes idle with at most ksmax waves. Segments
        // hold whole blocks (and q4_0 block pairs) so that lanes which share
        // data through DPP stay in one wave.
        constexpr int UPB = (F == Q4_0 || F == Q8_0_F16) ? 2 : Layout<F>::QK / Unit<F>::W;
        // QK_TUNE_GEMV_SLOT = 32 or 64 forces the slot width where it gives a plan
        const int slot_env = tuning(QK_TUNE_GEMV_SLOT);
        double best = 0.0;
        for (int pass = (slot_env == 32 || slot_env == 64) ? 0 : 1; pass < 2 && best == 0.0; pass++) {
            for (int sh = 6; sh >= 5; sh--) {
                const int L = 1 << sh;
                if (pass == 0 && L != slot_env) continue;
                const int ks = (int)((U + L - 1) / L);
                if (ks > ksmax) continue;
                int uw = (int)((U + ks - 1) / ks);
                uw = (uw + UPB - 1) / UPB * UPB;
                if (uw > L) continue;
                const double util = (double)U / (double)(ks * L);
                if (util > best + 1e-9) {
                    best = util;
                    p.KS = ks;
                    p.Uw = uw;
                    p.Lshift = sh;
                    p.RP = 64 / L;
                }
            }
        }
    }
    const int nwr_env = tuning(QK_TUNE_GEMV_NWR);
    // waves per workgroup: 4 (more, for wide rows, measured slower), or KS
    // when a row takes more than 4 waves
    const int wmax = cols > kRegStageCols ? 8 : 4;  // the kernels' launch bounds (512 / 256 threads)
    p.NWR = nwr_env > 0 && nwr_env * p.KS <= wmax ? nwr_env : (4 / p.KS > 0 ? 4 / p.KS : 1);
    if (cols <= kRegStageCols)
        while (32 * 64 * p.KS * p.NWR < cols) p.NWR++;  // enough threads to stage x
    p.ksmul = 65536 / p.KS + 1;
    return p;
}

}  // namespace qk
