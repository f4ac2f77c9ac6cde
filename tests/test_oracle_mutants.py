"""Planted mistakes in the oracle must each fail at least one pin.

Each case copies ``oracle/lowbit_oracle.c`` to a temporary directory, applies
one plausible mistake (a dropped term, a wrong sign or index, the wrong
rounding rule, a transposed operand), compiles it with the oracle's own
flags, and runs every pin against that broken build.  The mistake is planted
in the oracle only, on the CPU.
"""
import os
import subprocess

import pytest

import pins
from oracle import Oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "lowbit_oracle.c")

MUTANTS = {
    "codes_round_half_away": ("float t = nearbyintf(v / s);", "float t = roundf(v / s);"),
    "zero_round_half_away": ("float zf = nearbyintf(-lo / s);", "float zf = roundf(-lo / s);"),
    "zero_wrong_sign": ("float zf = nearbyintf(-lo / s);", "float zf = nearbyintf(lo / s);"),
    "scale_not_stored_as_fp16": ("float s = (float)orc_f16_to_f64(s16);",
                                 "float s = (s32 == 0.0f) ? 1.0f : s32;"),
    "levels_off_by_one": ("const int M = (1 << bits) - 1;", "const int M = (1 << bits);"),
    "no_upper_clamp": ("if (q > M) q = M;", "if (q > M + 1) q = M;"),
    "min_starts_at_zero": ("float lo = (float)orc_f16_to_f64(wg[0]);", "float lo = 0.0f;"),
    "group_scan_drops_last": ("for (int64_t k = 1; k < g; ++k) {",
                              "for (int64_t k = 1; k < g - 1; ++k) {"),
    "pack_drops_straddle": ("if (off + bits > 32) row[wi + 1] |= q >> (32 - off);", ""),
    "pack_msb_first": ("row[wi] |= q << off;", "row[wi] |= q << (32 - bits - off);"),
    "dequant_adds_zero": ("(double)((int64_t)codes[n * K + k] - (int64_t)zeros[n * G + j])",
                          "(double)((int64_t)codes[n * K + k] + (int64_t)zeros[n * G + j])"),
    "dequant_wrong_group": ("int64_t j = k / g;", "int64_t j = k % G;"),
    "f16_round_ties_away": ("double m = nearbyint(ldexp(a, 10 - e));",
                            "double m = round(ldexp(a, 10 - e));"),
    "f16_decode_wrong_bias": ("v = ldexp((double)(1024 + f), e - 25);",
                              "v = ldexp((double)(1024 + f), e - 24);"),
    "matmul_transposed": ("* deq[n * K + k];", "* deq[k * N + n];"),
    "dequant_rounded_to_fp16": ("deq[n * K + k] = qz * s;",
                                "deq[n * K + k] = orc_f16_to_f64(orc_f64_to_f16(qz * s));"),
    "gptq_deq_rounded_to_fp16": ("const double deq = (double)(q - z) * s;",
                                 "const double deq = orc_f16_to_f64(orc_f64_to_f16((double)(q - z) * s));"),
    "sym_divisor_power_of_two": ("const int qmax = (1 << (bits - 1)) - 1;",
                                 "const int qmax = (1 << (bits - 1));"),
    "sym_no_absolute_value": ("float a = fabsf((float)orc_f16_to_f64(wr[k]));",
                              "float a = (float)orc_f16_to_f64(wr[k]);"),
    "sym_zero_off_by_one": ("const int32_t z = 1 << (bits - 1);",
                            "const int32_t z = (1 << (bits - 1)) - 1;"),
    "sym_round_half_away": ("float r = nearbyintf(v / sc);", "float r = roundf(v / sc);"),
    "meta_zero_not_sign_extended": ("zeros[i] = (int32_t)(int16_t)(uint16_t)(meta[i] >> 16);",
                                    "zeros[i] = (int32_t)(meta[i] >> 16);"),
    "meta_no_saturation": ("if (z > 32767) { z = 32767; ++saturated; }", ""),
    "meta_fields_swapped": ("meta[i] = (uint32_t)scales[i] | (zfield << 16);",
                            "meta[i] = zfield | ((uint32_t)scales[i] << 16);"),
    "gptq_update_sign": ("for (int64_t j = i + 1; j < K; ++j) cur[n * K + j] -= err * hinv[i * K + j];",
                         "for (int64_t j = i + 1; j < K; ++j) cur[n * K + j] += err * hinv[i * K + j];"),
    "gptq_no_downdate": ("for (int64_t k = i + 1; k < K; ++k) hinv[j * K + k] -= f * hinv[i * K + k];",
                         ""),
    "gptq_err_not_scaled": ("const double err = (v - deq) / hii;", "const double err = (v - deq);"),
    "gptq_sym_clamp_from_zero": ("const int64_t minq = sym ? 1 : 0;", "const int64_t minq = 0;"),
    "hessian_damp_not_mean": ("const double add = damp * tr / (double)K;",
                              "const double add = damp * tr;"),
    "hessian_missing_factor_two": ("H[i] = 2.0 * H[i] / (double)n;", "H[i] = H[i] / (double)n;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    src = tmp_path / "lowbit_oracle.c"
    src.write_text(text.replace(old, new))
    (tmp_path / "lowbit_oracle.h").write_text(
        open(os.path.join(ROOT, "oracle", "lowbit_oracle.h")).read())
    so = tmp_path / f"mutant_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", str(so), str(src), "-lm"], check=True)
    mutant = Oracle(str(so))
    failed = []
    for check in pins.ALL_CHECKS:
        try:
            check(mutant)
        except AssertionError:
            failed.append(check.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
