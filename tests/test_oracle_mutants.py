"""Planted mistakes: each is a one-line change to a copy of the oracle source,
compiled on the CPU; the pin battery must reject every one of them."""
import os

import pytest

import oracle as O
import oracle_pins

MUTANTS = {
    "e2m1_bias": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e2m1_sign_dropped": ("    return s ? -v : v;\n}\n\n/* NVFP4 subblock", "    return v;\n}\n\n/* NVFP4 subblock"),
    "ue4m3_subnormal": ("return ldexp((double)m, -9);", "return ldexp((double)m, -10);"),
    "ue4m3_bias": ("return ldexp(1.0 + m / 8.0, e - 7);", "return ldexp(1.0 + m / 8.0, e - 8);"),
    "f16_tie_rule": ("if (rem > 0x1000u || (rem == 0x1000u && (res & 1u)))", "if (rem >= 0x1000u)"),
    "f16_subnormal_shift": ("int shift = 14 - e;", "int shift = 13 - e;"),
    "q8_round_half_away": ("float r = rintf(t);", "float r = roundf(t);"),
    "q8_divide_by_f16": ("float t = xb[j] / d;", "float t = xb[j] / (float)nvqo_f16_to_f64(nvqo_f32_to_f16(d));"),
    "q8_zero_scale_guard": ("if (d != 0.0f) {", "if (amax != 0.0f) {"),
    "q8_bsum_offset": ("bsum16[m * (K / 16) + 2 * b + h] = (int16_t)s;", "bsum16[m * (K / 16) + 2 * b + (1 - h)] = (int16_t)s;"),
    "isums_index": ("acc += l * (int32_t)q[m * K + k];", "acc += l * (int32_t)q[m * K + (k ^ 1)];"),
    "act_scale_index": ("a[k] = nvqo_f16_to_f64(d16[k / 32]) * (double)q[k];", "a[k] = nvqo_f16_to_f64(d16[k / 16 % (K / 32)]) * (double)q[k];"),
    "weight_scale_index": ("w[k] = (double)w_scale * nvqo_ue4m3(scales[k / 16]) * nvqo_e2m1(codes[k]);",
                           "w[k] = (double)w_scale * nvqo_ue4m3(scales[k / 32]) * nvqo_e2m1(codes[k]);"),
    "routed_token_row": ("q + m * K, d16 + m * (K / 32), 1, N, K, cols, ncols, yj, aj);",
                         "q, d16 + m * (K / 32), 1, N, K, cols, ncols, yj, aj);"),
    "routed_expert_scale": ("scales + e * N * (K / 16), w_scales[e],", "scales + e * N * (K / 16), w_scales[a % E],"),
    "routed_expert_codes": ("nvqo_matmul_nvfp4(codes + e * N * K,", "nvqo_matmul_nvfp4(codes + (E - 1 - e) * N * K,"),
    "q4_1_offset_dropped": ("w[k] = nvqo_f16_to_f64(dw[k / 32]) * (double)qw[k] + nvqo_f16_to_f64(mw[k / 32]);",
                            "w[k] = nvqo_f16_to_f64(dw[k / 32]) * (double)qw[k];"),
    "q4_k_first_subblock_scale": ("int64_t s = k / 256, j = k / 32;", "int64_t s = k / 256, j = (k / 256) * 8;"),
    "q4_k_min_sign": ("             - nvqo_f16_to_f64(dmin[s]) * (double)mn[j];", "             + nvqo_f16_to_f64(dmin[s]) * (double)mn[j];"),
    "q4_k_scales_swapped": ("w[k] = nvqo_f16_to_f64(d[s]) * (double)sc[j] * (double)qw[k]", "w[k] = nvqo_f16_to_f64(dmin[s]) * (double)sc[j] * (double)qw[k]"),
    "iq4_xs_table_index": ("acc += (int32_t)table[qw[n * K + k]] * (int32_t)q[m * K + k];",
                           "acc += (int32_t)table[qw[n * K + k] ^ 1] * (int32_t)q[m * K + k];"),
    "iq4_xs_scale_offset": ("(double)((int)ls[k / 32] - 32)", "(double)((int)ls[k / 32] - 31)"),
    "iq4_xs_code_not_looked_up": ("* (double)table[qw[k]];", "* (double)qw[k];"),
    "q5_k_fifth_bit_dropped": ("w[k] = scale * (double)qw[k] - offset;", "w[k] = scale * (double)(qw[k] & 15) - offset;"),
    "q5_k_min_per_super_block": ("double offset = nvqo_f16_to_f64(dmin[k / 256]) * (double)mn[k / 32];",
                                 "double offset = nvqo_f16_to_f64(dmin[k / 256]) * (double)mn[(k / 256) * 8];"),
    "q6_k_offset_31": ("* (double)((int)qw[k] - 32);", "* (double)((int)qw[k] - 31);"),
    "q6_k_scale_per_32": ("(double)sc[k / 16] * (double)((int)qw[k] - 32)", "(double)sc[k / 32] * (double)((int)qw[k] - 32)"),
    "q6_k_isums_unsigned": ("acc += ((int32_t)qw[n * K + k] - 32) * (int32_t)q[m * K + k];",
                            "acc += (int32_t)qw[n * K + k] * (int32_t)q[m * K + k];"),
    "transposed_product": ("dot_rows(w, a + m * K, K, &y[m * ncols + j],\n                     abs_wa ? &abs_wa[m * ncols + j] : NULL);\n    }\n    free(w);\n    free(a);\n}\n\n/* Expert-routed",
                           "dot_rows(w, a + m * K, K, &y[j * M + m],\n                     abs_wa ? &abs_wa[m * ncols + j] : NULL);\n    }\n    free(w);\n    free(a);\n}\n\n/* Expert-routed"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(O.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique/found"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = str(tmp_path / "libmutant.so")
    O.build(out=lib, src=str(mpath))
    results = oracle_pins.battery(O.Oracle(lib))
    failed = [n for n, ok, _ in results if not ok]
    assert failed, f"mutant {name} passed every pin"
