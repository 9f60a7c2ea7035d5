"""Plant plausible mistakes in a copy of the oracle (on the CPU) and show
that the pins catch every one of them.  A mutant that passes every pin
would mean the pins cannot tell that mistake from the spec's rule."""
import os

import pytest

import pins
from oracle import oracle as orc

SRC = os.path.join(os.path.dirname(orc.__file__), "qmv_oracle.c")

# (name, text in the source, replacement, occurrence to replace or None = all)
# Not listed: widening the Q8 clamp to -128.  For finite input |x * id| is at
# most 127 * (1 + 2^-23)^2, so trunc(x * id +- 0.5) never leaves [-127, 127]
# and that edit cannot change any output (an equivalent mutant).
MUTANTS = [
    ("round_by_division", "float v = xb[i] * id;\n            float t = v + copysignf(0.5f, xb[i]);\n            int qi = (int)truncf(t);\n            if (qi > 127)",
     "float v = xb[i] / db;\n            float t = v + copysignf(0.5f, xb[i]);\n            int qi = (int)truncf(t);\n            if (qi > 127)", 1),
    ("id_from_d", "float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;", "float id = (amax != 0.0f) ? 1.0f / db : 0.0f;", 1),
    ("fused_multiply_add", "float v = xb[i] * id;\n            float t = v + copysignf(0.5f, xb[i]);\n            int qi = (int)truncf(t);\n            if (qi > 127)",
     "float t = fmaf(xb[i], id, copysignf(0.5f, xb[i]));\n            int qi = (int)truncf(t);\n            if (qi > 127)", 1),
    ("round_half_even", "int qi = (int)truncf(t);\n            if (qi > 127)", "int qi = (int)rintf(v);\n            (void)t;\n            if (qi > 127)", 1),
    ("truncate_only", "float t = v + copysignf(0.5f, xb[i]);\n            int qi = (int)truncf(t);\n            if (qi > 127)",
     "float t = v;\n            int qi = (int)truncf(t);\n            if (qi > 127)", 1),
    ("scale_128", "float db = amax / 127.0f;", "float db = amax / 128.0f;", 1),
    ("signed_max", "float a = fabsf(xb[i]);\n            if (a > amax)\n                amax = a;\n        }\n        float db = amax / 127.0f;",
     "float a = xb[i];\n            if (a > amax)\n                amax = a;\n        }\n        float db = amax / 127.0f;", 1),
    ("q4_nibbles_swapped", "(i < QK / 2) ? (blk[i] & 0x0F) : (blk[i - QK / 2] >> 4)", "(i < QK / 2) ? (blk[i] >> 4) : (blk[i - QK / 2] & 0x0F)", 1),
    ("q4_interleaved", "(i < QK / 2) ? (blk[i] & 0x0F) : (blk[i - QK / 2] >> 4)", "(i % 2 == 0) ? (blk[i / 2] & 0x0F) : (blk[i / 2] >> 4)", 1),
    ("q4_offset_7", "return nib - 8;", "return nib - 7;", 1),
    ("q4_pack_interleaved", "q[b * (QK / 2) + j] = (uint8_t)(nib[j] | (nib[j + QK / 2] << 4));",
     "q[b * (QK / 2) + j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));", 1),
    ("q4_scale_8", "float db = amax / 7.0f;", "float db = amax / 8.0f;", 1),
    ("drop_last_block", "for (int32_t b = 0; b < nb; ++b) {\n        const int8_t *w = wq + (int64_t)r * cols + (int64_t)b * QK;\n        const int8_t *xv = xq + (int64_t)b * QK;\n        int32_t sumi = 0;",
     "for (int32_t b = 0; b < nb - 1; ++b) {\n        const int8_t *w = wq + (int64_t)r * cols + (int64_t)b * QK;\n        const int8_t *xv = xq + (int64_t)b * QK;\n        int32_t sumi = 0;", 1),
    ("dx_wrong_index", "t = t * xd[b];", "t = t * xd[r % nb];", None),
    ("dw_transposed", "float t = (float)sumi * wd[(int64_t)r * nb + b];", "float t = (float)sumi * wd[(int64_t)b * nb + r % nb];", None),
    ("drop_dx", "t = t * xd[b];", "t = t * 1.0f;", None),
    ("acc_overwrite", "s = s + t;", "s = t;", None),
    ("sum_sign", "sumi += (int32_t)q4_elem(blk, i) * (int32_t)xv[i];", "sumi -= (int32_t)q4_elem(blk, i) * (int32_t)xv[i];", None),
    ("y_relative_index", "y[r] = row_q8(wq, wd, cols, xq, xd, r);", "y[r - r0] = row_q8(wq, wd, cols, xq, xd, r);", 1),
    ("gemm_x_stride", "xq + (int64_t)i * cols, xd + (int64_t)i * nb, r0, r1);", "xq + (int64_t)i * cols, xd, r0, r1);", None),
    ("rms_block_left_to_right", "bs[b] = pairwise_sum(sq, QK);",
     "float t = 0.0f;\n        for (int i = 0; i < QK; ++i)\n            t += sq[i];\n        bs[b] = t;", 1),
    ("rms_blocks_left_to_right", "float ss = pairwise_sum(bs, p);",
     "float ss = 0.0f;\n    for (int64_t b = 0; b < p; ++b)\n        ss += bs[b];", 1),
    ("rms_no_eps", "float inv = 1.0f / sqrtf(mean + eps);", "float inv = 1.0f / sqrtf(mean);", 1),
    ("rms_n_minus_1", "float mean = ss / (float)n;", "float mean = ss / (float)(n - 1);", 1),
    ("rms_no_weight", "o[j] = w[j] * (inv * x[j]);", "o[j] = inv * x[j];", 1),
    ("rms_abs_not_square", "sq[i] = x[b * QK + i] * x[b * QK + i];", "sq[i] = fabsf(x[b * QK + i]);", 1),
    ("silu_sign", "float s = 1.0f / (1.0f + expf(-v));", "float s = 1.0f / (1.0f + expf(v));", 1),
    ("silu_no_gate", "o[j] = v * u[j];", "o[j] = v;", 1),
    ("silu_sigmoid_only", "v = v * s;\n        o[j] = v * u[j];", "v = s;\n        o[j] = v * u[j];", 1),
    ("rms_weight_shift", "o[j] = w[j] * (inv * x[j]);", "o[j] = w[(j + 1) % n] * (inv * x[j]);", 1),
    ("b128_max_first_32", "for (int i = 0; i < BL; ++i) {\n            float a = fabsf(xb[i]);",
     "for (int i = 0; i < 32; ++i) {\n            float a = fabsf(xb[i]);", 1),
    ("b128_scale_128", "float db = amax / 127.0f;\n        float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;\n        for (int i = 0; i < BL; ++i) {",
     "float db = amax / 128.0f;\n        float id = (amax != 0.0f) ? 127.0f / amax : 0.0f;\n        for (int i = 0; i < BL; ++i) {", 1),
    ("zp_dropped", "s += (int32_t)(zp_code(row, bits, e) - zp) * (int32_t)xq[e];", "s += (int32_t)zp_code(row, bits, e) * (int32_t)xq[e];", 1),
    ("zp_default_127", "return 1 << (bits - 1);", "return (1 << (bits - 1)) - 1;", 1),
    ("zp_nibbles_swapped", "return (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);", "return (i % 2 == 0) ? (byte >> 4) : (byte & 0x0F);", 1),
    ("zp_nibbles_halves", "uint8_t byte = row[i / 2];\n    return (i % 2 == 0) ? (byte & 0x0F) : (byte >> 4);",
     "uint8_t byte = row[(i / 128) * 64 + (i % 64)];\n    return (i % 128 < 64) ? (byte & 0x0F) : (byte >> 4);", 1),
    ("zp_q4_row_stride", "const uint8_t *row = wq + (int64_t)r * (bits == 8 ? cols : cols / 2);", "const uint8_t *row = wq + (int64_t)r * cols / 2;", 1),
    ("zp_per_block_only", "return wzp[(int64_t)r * nb + b];", "return wzp[b];", 1),
    ("zp_sign", "s += (int32_t)(zp_code(row, bits, e) - zp) * (int32_t)xq[e];", "s += (int32_t)(zp - zp_code(row, bits, e)) * (int32_t)xq[e];", 1),
    ("b256_max_first_32", "for (int i = 0; i < SBK; ++i) {\n            float a = fabsf(xb[i]);",
     "for (int i = 0; i < 32; ++i) {\n            float a = fabsf(xb[i]);", 1),
    ("q4k_nibbles_swapped", "return (i < 16) ? (sub[i] & 0x0F) : (sub[i - 16] >> 4);",
     "return (i < 16) ? (sub[i] >> 4) : (sub[i - 16] & 0x0F);", 1),
    ("q4k_nibbles_interleaved", "return (i < 16) ? (sub[i] & 0x0F) : (sub[i - 16] >> 4);",
     "return (i % 2 == 0) ? (sub[i / 2] & 0x0F) : (sub[i / 2] >> 4);", 1),
    ("q4k_offset_8", "dot += (int64_t)q4k_nib(sub, i) * xv[i];", "dot += (int64_t)(q4k_nib(sub, i) - 8) * xv[i];", 1),
    ("q4k_no_min", "float v = t - u;", "float v = t;", 1),
    ("q4k_min_sign", "float v = t - u;", "float v = t + u;", 1),
    ("q4k_d_dmin_swapped", "float t = (float)s1 * d[(int64_t)r * nk + k];\n            float u = (float)s2 * dmin[(int64_t)r * nk + k];",
     "float t = (float)s1 * dmin[(int64_t)r * nk + k];\n            float u = (float)s2 * d[(int64_t)r * nk + k];", 1),
    ("q4k_scale_per_superblock", "a += (int64_t)sc[(int64_t)r * nsub + sb] * dot;", "a += (int64_t)sc[(int64_t)r * nsub + k * 8] * dot;", 1),
    ("q4k_min_times_nibbles", "qs += xv[i];", "qs += (int64_t)q4k_nib(sub, i) * xv[i];", 1),
    ("q4k_min_from_scale", "m += (int64_t)mn[(int64_t)r * nsub + sb] * qs;", "m += (int64_t)sc[(int64_t)r * nsub + sb] * qs;", 1),
    ("q4k_dx_dropped", "v = v * xd[k];", "v = v * 1.0f;", 1),
    ("zp_acc_skips_last", "for (int32_t b = 0; b < nb; ++b) {\n            int32_t sumi = zp_block_sum(bits, wq, wzp, cols, xq, r, b);\n            float t",
     "for (int32_t b = 0; b + 1 < nb; ++b) {\n            int32_t sumi = zp_block_sum(bits, wq, wzp, cols, xq, r, b);\n            float t", 1),
]


def _apply(src, old, new, count):
    assert old in src, "mutation site not found"
    return src.replace(old, new) if count is None else src.replace(old, new, count)


@pytest.mark.parametrize("name,old,new,count", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, name, old, new, count):
    with open(SRC) as f:
        src = f.read()
    mutated = _apply(src, old, new, count)
    assert mutated != src
    so = orc.build_variant(mutated, str(tmp_path / f"mut_{name}.so"))
    with orc.use_build(so):
        failed = pins.failing_checks()
    assert failed, f"no pin catches the planted mistake '{name}'"
