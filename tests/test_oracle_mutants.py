"""The oracle's pins must reject plausible mistakes.

Each case plants one mistake in a temporary copy of the oracle's C source (on the CPU),
builds it, routes the oracle through it and runs the pins: at least one must fail.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_formats as tf
from tests import test_oracle_pipeline as tp
from tests import test_oracle_quantizer as tq
from tests import test_oracle_codec as tc
from tests import test_oracle_fixed as tfx
from tests import test_oracle_group as tg

MUTANTS = {
    "ties_away_from_zero": ("float v = rintf(x * inv);", "float v = roundf(x * inv);"),
    "scale_128": ("return s > 0.0f ? 127.0f / s : 0.0f;", "return s > 0.0f ? 128.0f / s : 0.0f;"),
    "threshold_not_strict": ("dt)) > tau) flag[j] = 1;", "dt)) >= tau) flag[j] = 1;"),
    "row_scale_over_all_columns": ("            if (is_out[j]) continue;\n", ""),
    "row_scale_used_for_column": ("float yi = (cf * ri) * cn;", "float yi = (cf * ri) * ri;"),
    "outlier_part_dropped": ("float v = yi + yo;", "float v = yi;"),
    "outlier_part_sign": ("f = f + p;", "f = f - p;"),
    "outlier_gather_index": ("XO[i * nO + t] = row[O[t]];", "XO[i * nO + t] = row[t];"),
    "outlier_weight_index": ("(float)Wq[n * K + O[t]];", "(float)Wq[n * K + t];"),
    "fp16_round_half_up": ("r += 0xfffu + ((r >> 13) & 1u);", "r += 0x1000u;"),
    "weight_transposed": ("Wq[n * K + k] = orc_quantize(orc_to_f32(W[k * N + n], dt), inv[n - nb]);",
                          "Wq[n * K + k] = orc_quantize(orc_to_f32(W[(k * N + n) % (K * N)], dt), inv[(n * 7) % (ne - nb)]);"),
    "int_gemm_transposed": ("const int8_t* w = Wq + n * K;", "const int8_t* w = Wq + ((n + 1) % N) * K;"),
    "codec_block_end_off_by_one": ("int64_t lo = b * block, hi = lo + block < n ? lo + block : n;\n        float s = 0.0f;",
                                   "int64_t lo = b * block, hi = lo + block - 1 < n ? lo + block - 1 : n;\n        float s = 0.0f;"),
    "codec_scale_first_element": ("            if (a > s) s = a;\n        }\n        absmax[b] = s;",
                                  "            if (a > s && i == lo) s = a;\n        }\n        absmax[b] = s;"),
    "codec_decode_128": ("float step = absmax[b] / 127.0f;", "float step = absmax[b] / 128.0f;"),
    "fixed_outlier_part_scaled": ("float v = y_int + F[r * N + n];", "float v = y_int + cn * F[r * N + n];"),
    "fixed_scale_over_all_rows": ("            if (is_out[k]) continue;\n            float a = fabsf(orc_to_f32(W[k * N + n], dt));",
                                  "            float a = fabsf(orc_to_f32(W[k * N + n], dt));"),
    "fixed_rows_from_codes": ("WO[n * nO + t] = W[(int64_t)O[t] * N + n];",
                              "WO[n * nO + t] = orc_from_f32((float)Wq[n * K + O[t]], dt);"),
    "group_row_scale_over_whole_row": ("            const uint16_t* xs = X + i * K + g * G;\n            float s = 0.0f;\n            for (int64_t k = 0; k < G; ++k) {",
                                       "            const uint16_t* xs = X + i * K + g * G;\n            float s = 0.0f;\n            for (int64_t k = -g * G; k < K - g * G; ++k) {"),
    "group_weight_boundary_shift": ("            for (int64_t k = g * G; k < (g + 1) * G; ++k) {\n                float a = fabsf(orc_to_f32(W[k * N + n], dt));",
                                    "            for (int64_t k = g * G; k < (g + 1) * G && k + 1 < K; ++k) {\n                float a = fabsf(orc_to_f32(W[k * N + n], dt));"),
    "group_sum_scaled_once": ("                float term = ((float)cg * rg) * cng;\n                acc = acc + term;",
                              "                float term = ((float)cg * rg) * cng;\n                acc = g == 0 ? term : acc + (float)cg * (acc / (float)cg);"),
}

PINS = [
    tf.test_narrowing_round_to_nearest_even,
    tq.test_quantizer_ties_go_to_even,
    lambda: tq.test_quantizer_exact_on_power_of_two_scales("fp16", 0),
    tp.test_outlier_threshold_is_strict,
    tp.test_row_scale_excludes_outlier_columns_not_just_large_values,
    tp.test_row_quantization_brute_force,
    tp.test_weight_quantization_brute_force,
    tp.test_int_gemm_against_numpy_int64,
    tp.test_epilogue_closed_form_on_lattice,
    tp.test_outlier_gemm_exact_on_integers_and_close_to_float64,
    lambda: tc.test_codec_lattice_round_trip_is_exact(64),
    lambda: tc.test_codec_blocks_use_the_scalar_quantizer(64),
    lambda: tc.test_codec_error_bound_and_range(256),
    tfx.test_fixed_lattice_closed_form,
    tfx.test_fixed_weight_conversion_uses_the_scalar_quantizer,
    tfx.test_fixed_all_columns_is_the_16bit_product,
    tg.test_group_lattice_closed_form,
    lambda: tg.test_group_codes_use_the_scalar_quantizer("fp16", 64),
    tg.test_group_fp32_sum_within_its_bound,
]


def _run_pin(pin):
    import inspect
    args = inspect.signature(pin).parameters
    if "dt" in args:
        for dt in ("fp16", "bf16"):
            pin(dt)
    else:
        pin()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, name
    d = tmp_path / "m"
    d.mkdir()
    (d / "oracle.c").write_text(src.replace(old, new))
    (d / "oracle.h").write_text(open(os.path.join(oracle.HERE, "oracle.h")).read())
    lib = str(d / "liborc_mutant.so")
    subprocess.check_call(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared",
                           "-o", lib, str(d / "oracle.c"), "-lm"])
    failed = []
    with oracle.use_library(lib):
        for pin in PINS:
            try:
                _run_pin(pin)
            except (AssertionError, OverflowError, ValueError, IndexError):
                failed.append(getattr(pin, "__name__", "pin"))
    assert failed, "no pin rejects the mutant " + name
