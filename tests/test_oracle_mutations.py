"""Mutation checks: plausible mistakes planted in a copy of the oracle's
source (on the CPU) must each make at least one pin fail. This shows the
pins can fail, including on the exact bug the Q6_K debugging page records
(one scale per 32 weights instead of per 16)."""
import os

import pytest

import oracle
import pins

MUTATIONS = {
    # the page's bug: the Q6_K scale index does not advance every 16 weights
    "q6k_scale_per_32": ("const int is_l = is + l / 16;", "const int is_l = is;"),
    # Q4_K straddling sub-blocks 4..7 take the scale's high bits from byte j
    "q4k_straddle_scale_byte": ("((packed[j - 4] >> 6) << 4)", "((packed[j] >> 6) << 4)"),
    # ... or the min's high bits from byte j-4
    "q4k_straddle_min_byte": ("m = (packed[j + 4] >> 4) | ((packed[j] >> 6) << 4);",
                              "m = (packed[j + 4] >> 4) | ((packed[j - 4] >> 6) << 4);"),
    "q4k_nibbles_swapped": ("half ? (byte >> 4) : (byte & 0xF)", "half ? (byte & 0xF) : (byte >> 4)"),
    "q4k_dmin_offset": ("rd_u16le(blk + 2)", "rd_u16le(blk + 0)"),
    "q4k_min_sign": ("out[64 * g + 32 * half + l] = t - m;", "out[64 * g + 32 * half + l] = t + m;"),
    "q6k_no_offset": ("const int q = (low4 | (high2 << 4)) - 32;", "const int q = (low4 | (high2 << 4));"),
    "q6k_qh_shift": ("(qh[32 * h + l] >> (2 * k)) & 3", "(qh[32 * h + l] >> k) & 3"),
    "q6k_quarter_source": ("ql[64 * h + 32 * (k & 1) + l]", "ql[64 * h + 32 * (k >> 1) + l]"),
    "q4_0_interleaved": ("out[j] = d * (float)((qs[j] & 0xF) - 8);\n        out[j + 16] = d * (float)((qs[j] >> 4) - 8);",
                         "out[2 * j] = d * (float)((qs[j] & 0xF) - 8);\n        out[2 * j + 1] = d * (float)((qs[j] >> 4) - 8);"),
    "q4_0_no_offset": ("out[j + 16] = d * (float)((qs[j] >> 4) - 8);", "out[j + 16] = d * (float)((qs[j] >> 4));"),
    "fp16_big_endian": ("return (uint16_t)(p[0] | (p[1] << 8));", "return (uint16_t)(p[1] | (p[0] << 8));"),
    "fp16_subnormal_scale": ("v = ldexpf((float)f, -24);", "v = ldexpf((float)f, -25);"),
    "fp16_bias": ("v = ldexpf((float)(1024 + f), e - 25);", "v = ldexpf((float)(1024 + f), e - 24);"),
    "q8_0_scale_as_fp16": ("const float s = f32_from_bits(rd_u32le(blk));", "const float s = qko_half_to_float(rd_u16le(blk));"),
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
