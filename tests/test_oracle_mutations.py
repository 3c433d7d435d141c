"""Mutation checks: plausible mistakes planted in a copy of the oracle's
source (on the CPU) must each make at least one pin fail. This shows the
pins can fail, including on the exact bug the Q6_K debugging page records
(one scale per 32 weights instead of per 16)."""
import os

import pytest

import oracle
import pins

MUTATIONS = {
    # the page's bug: one Q6_K scale per 32 weights (the scale of the first 16
    # of each 32 used for all of them) instead of one per 16
    "q6k_scale_per_32": ("float w = d * (float)scales[i / 16];", "float w = d * (float)scales[2 * (i / 32)];"),
    # Q4_K straddling sub-blocks 4..7 take the top bits of the scale from the
    # min's byte and those of the min from the scale's byte
    "q4k_straddle_top_bits_swapped": ("const int top2 = packed_bits(packed, first + 8 * (j - 4) + 6, 2);",
                                      "const int top2 = packed_bits(packed, 32 - first + 8 * (j - 4) + 6, 2);"),
    # ... or index the byte of the top bits by j instead of j - 4
    "q4k_straddle_top_bits_byte": ("const int top2 = packed_bits(packed, first + 8 * (j - 4) + 6, 2);",
                                   "const int top2 = packed_bits(packed, first + 8 * j + 6, 2);"),
    # ... or swap the low nibbles of scale and min in bytes 8..11
    "q4k_straddle_low_nibbles": ("64 + 8 * (j - 4) + (is_min ? 4 : 0), 4);", "64 + 8 * (j - 4) + (is_min ? 0 : 4), 4);"),
    # sub-blocks 0..3 read all 8 bits of their byte
    "q4k_field_width": ("if (j < 4) return packed_bits(packed, first + 8 * j, 6);",
                        "if (j < 4) return packed_bits(packed, first + 8 * j, 8);"),
    "q4k_nibbles_swapped": ("const int q = half ? (byte >> 4) : (byte & 0xF);",
                            "const int q = half ? (byte & 0xF) : (byte >> 4);"),
    "q4k_dmin_offset": ("const float dmin = qko_half_to_float(rd_u16le(blk + 2));\n    const uint8_t *packed = blk + 4;\n"
                        "    const uint8_t *qs = blk + 16;",
                        "const float dmin = qko_half_to_float(rd_u16le(blk + 0));\n    const uint8_t *packed = blk + 4;\n"
                        "    const uint8_t *qs = blk + 16;"),
    "q4k_min_sign": ("const float m = dmin * mn[j];\n                out[64 * g + 32 * half + l] = t - m;",
                     "const float m = dmin * mn[j];\n                out[64 * g + 32 * half + l] = t + m;"),
    "q6k_no_offset": ("const int q = (low4 | (high2 << 4)) - 32;", "const int q = (low4 | (high2 << 4));"),
    "q6k_qh_shift": ("(qh[32 * h + l] >> (2 * k)) & 3", "(qh[32 * h + l] >> k) & 3"),
    "q6k_quarter_source": ("ql[64 * h + 32 * (k % 2) + l]", "ql[64 * h + 32 * (k / 2) + l]"),
    "q4_0_interleaved": ("out[j] = d * (float)((qs[j] & 0xF) - 8);\n        out[j + 16] = d * (float)((qs[j] >> 4) - 8);",
                         "out[2 * j] = d * (float)((qs[j] & 0xF) - 8);\n        out[2 * j + 1] = d * (float)((qs[j] >> 4) - 8);"),
    "q4_0_no_offset": ("out[j + 16] = d * (float)((qs[j] >> 4) - 8);", "out[j + 16] = d * (float)((qs[j] >> 4));"),
    "fp16_big_endian": ("return (uint16_t)(p[0] | (p[1] << 8));", "return (uint16_t)(p[1] | (p[0] << 8));"),
    "fp16_subnormal_scale": ("v = ldexpf((float)f, -24);", "v = ldexpf((float)f, -25);"),
    "fp16_bias": ("v = ldexpf((float)(1024 + f), e - 25);", "v = ldexpf((float)(1024 + f), e - 24);"),
    "q8_0_scale_as_fp16": ("const float s = f32_from_bits(rd_u32le(blk));", "const float s = qko_half_to_float(rd_u16le(blk));"),
    # the ggml-layout formats: plausible misreadings of each layout, among
    # them wrong field offsets and bit order, the kind of error the
    # K-quants page reports in picoLM's Q2_K and Q3_K readers
    "q8_0_f16_unsigned": ("const int8_t *q = (const int8_t *)(blk + 2);", "const uint8_t *q = (const uint8_t *)(blk + 2);"),
    "q8_0_f16_offset": ("const int8_t *q = (const int8_t *)(blk + 2);", "const int8_t *q = (const int8_t *)(blk + 4);"),
    "q5_1_high_bit": ("(qh >> (j + 16))", "(qh >> (j + 12))"),
    "q5_1_min_sign": ("out[j + 16] = t + m;", "out[j + 16] = t - m;"),
    "q5_1_d_m_swapped": ("const float m = qko_half_to_float(rd_u16le(blk + 2));",
                         "const float m = qko_half_to_float(rd_u16le(blk + 0));"),
    "q5k_qh_bit_per_group": ("const int q = low4 | (((qh[l] >> j) & 1) << 4);",
                             "const int q = low4 | (((qh[l] >> g) & 1) << 4);"),
    "q5k_qs_offset": ("const uint8_t *qs = blk + 48;", "const uint8_t *qs = blk + 16;"),
    "q2k_scale_nibble": ("float t = d * (float)(sb & 0xF);", "float t = d * (float)(sb >> 4);"),
    "q2k_header_in_front": ("const float d = qko_half_to_float(rd_u16le(blk + 80));",
                            "const float d = qko_half_to_float(rd_u16le(blk + 0));"),
    "q2k_bit_order": ("const int q = (qs[32 * h + l] >> (2 * j)) & 3;", "const int q = (qs[32 * h + l] >> (6 - 2 * j)) & 3;"),
    "q2k_scale_per_32": ("const uint8_t sb = scales[i / 16];", "const uint8_t sb = scales[i / 32];"),
    "q2k_half_offset": ("const int q = (qs[32 * h + l] >> (2 * j)) & 3;", "const int q = (qs[l] >> (2 * j)) & 3;"),
    "q3k_hmask_bit": ("(hmask[l] >> (4 * h + j)) & 1", "(hmask[l] >> j) & 1"),
    "q3k_scale_high_bits": ("(sp[8 + s % 4] >> (2 * (s / 4))) & 3", "(sp[8 + s / 4] >> (2 * (s % 4))) & 3"),
    "q3k_mask_sense": ("const int q = q2 - (hb ? 0 : 4);", "const int q = q2 - (hb ? 4 : 0);"),
    "q3k_scale_bias": ("sc[s] = (low4 | (high2 << 4)) - 32;", "sc[s] = (low4 | (high2 << 4));"),
    "q3k_scale_low_nibble": ("const int low4 = s < 8 ? (sp[s] & 0xF) : (sp[s - 8] >> 4);",
                             "const int low4 = s < 8 ? (sp[s] >> 4) : (sp[s - 8] & 0xF);"),
    # the decode step and the encoder
    "half_ties_up": ("if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;", "if (frac >= 0.5) r += 1.0;"),
    "half_subnormal_step": ("if (ulp_exp < -24) ulp_exp = -24;", "if (ulp_exp < -25) ulp_exp = -25;"),
    "rmsnorm_eps_outside_root": ("const double inv = 1.0 / sqrt(ss / (double)n + (double)eps);",
                                 "const double inv = 1.0 / (sqrt(ss / (double)n) + (double)eps);"),
    "rmsnorm_sum_not_mean": ("const double inv = 1.0 / sqrt(ss / (double)n + (double)eps);",
                             "const double inv = 1.0 / sqrt(ss + (double)eps);"),
    "rope_sign": ("v[2 * i] = (float)(x0 * (double)c[i] - x1 * (double)s[i]);",
                  "v[2 * i] = (float)(x0 * (double)c[i] + x1 * (double)s[i]);"),
    "rope_neox_pairs": ("const double x0 = v[2 * i], x1 = v[2 * i + 1];\n            v[2 * i] = (float)(x0 * (double)c[i] - x1 * (double)s[i]);\n            v[2 * i + 1] = (float)(x0 * (double)s[i] + x1 * (double)c[i]);",
                        "const double x0 = v[i], x1 = v[i + head_dim / 2];\n            v[i] = (float)(x0 * (double)c[i] - x1 * (double)s[i]);\n            v[i + head_dim / 2] = (float)(x0 * (double)s[i] + x1 * (double)c[i]);"),
    "rope_frequency": ("pow(base, -2.0 * (double)i / (double)head_dim)", "pow(base, -(double)i / (double)head_dim)"),
    "attention_unscaled": ("sc[t] = dot * scale;", "sc[t] = dot;"),
    "attention_kv_head_modulo": ("const int g = h / grp;", "const int g = h % n_kv;"),
    # the attention tolerance scale: signed instead of absolute values, or
    # not divided by the softmax sum
    "attention_absacc_signed": ("aa += sc[t] * fabs(v);", "aa += sc[t] * v;"),
    "attention_absacc_unnormalised": ("if (absacc) absacc[(int64_t)h * head_dim + i] = aa / sum;",
                                      "if (absacc) absacc[(int64_t)h * head_dim + i] = aa;"),
    "swiglu_sign": ("out[i] = gv / (1.0 + exp(-gv)) * (double)u[i];", "out[i] = gv / (1.0 + exp(gv)) * (double)u[i];"),
    "q8_0_divisor_128": ("const float d = amax / 127.0f;", "const float d = amax / 128.0f;"),
    "q8_0_round_to_even": ("blk[4 + j] = (uint8_t)(int8_t)roundf(t);", "blk[4 + j] = (uint8_t)(int8_t)rintf(t);"),
    "q4_0_offset_8": ("const float t0 = v[j] * id + 8.5f;", "const float t0 = v[j] * id + 8.0f;"),
    "q4_0_no_cap": ("if (c0 > 15) c0 = 15;", ""),
    "q4_0_scale_sign": ("const float d = m / -8.0f;", "const float d = m / 8.0f;"),
    "gemv_drops_last_column": ("for (int64_t c = 0; c < cols; c++) {\n            const double p = (double)w[c] * (double)x[c];",
                               "for (int64_t c = 0; c < cols - 1; c++) {\n            const double p = (double)w[c] * (double)x[c];"),
    "gemv_sign": ("const double p = (double)w[c] * (double)x[c];", "const double p = -(double)w[c] * (double)x[c];"),
    "gemm_bf16_shift": ("const uint32_t u = (uint32_t)h << 16;", "const uint32_t u = (uint32_t)h << 15;"),
    "gemm_row_stride": ("Y[m * rows + r] = s;", "Y[r * M + m] = s;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(oracle.SRC).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(before, after))
    lib = oracle.build(src=str(path), out=str(tmp_path / "libmutant.so"))
    failed = pins.failing_pins(oracle.Oracle(lib))
    assert failed, f"mutation {name} passed every pin"


def test_real_oracle_passes_every_pin(orc):
    assert pins.failing_pins(orc) == []
