"""Mutation check of the oracle's pins.

Each case below plants one plausible mistake in a temporary copy of the
oracle's C source (a dropped term, a wrong sign or index, a transposed operand,
a wrong rounding), builds it on the CPU, and runs the pins against it.  Every
mutant must fail at least one pin; otherwise the pins would not notice that
mistake in the real oracle."""
import os

import numpy as np
import pytest

import oracle
import pins

MUTANTS = {
    "gate_dropped": ("float s = gate_or_null ? fmaf(bf16_to_f32(*gate_or_null), xv, r) : r + xv;",
                     "float s = r + xv;"),
    "gate_scales_residual": ("float s = gate_or_null ? fmaf(bf16_to_f32(*gate_or_null), xv, r) : r + xv;",
                             "float s = gate_or_null ? fmaf(bf16_to_f32(*gate_or_null), r, xv) : r + xv;"),
    "residual_product_rounded_first": (
        "float s = gate_or_null ? fmaf(bf16_to_f32(*gate_or_null), xv, r) : r + xv;",
        "float s = gate_or_null ? r + bf16_to_f32(*gate_or_null) * xv : r + xv;"),
    "norm_of_x_not_residual": ("h[c] = orc_bf16_to_f64(ro);",
                               "h[c] = orc_bf16_to_f64(x[k]);"),
    "modulation_sign": ("n * (1.0 + orc_bf16_to_f64(scale_row[c]))",
                        "n * (1.0 - orc_bf16_to_f64(scale_row[c]))"),
    "scale_shift_swapped": ("n * (1.0 + orc_bf16_to_f64(scale_row[c])) + orc_bf16_to_f64(shift_row[c])",
                            "n * (1.0 + orc_bf16_to_f64(shift_row[c])) + orc_bf16_to_f64(scale_row[c])"),
    "modulation_without_one": ("n * (1.0 + orc_bf16_to_f64(scale_row[c]))",
                               "n * (orc_bf16_to_f64(scale_row[c]))"),
    "unbiased_variance": ("double var = sq / (double)D;", "double var = sq / (double)(D - 1);"),
    "eps_outside_sqrt": ("double rho = 1.0 / sqrt(var + eps);",
                         "double rho = 1.0 / (sqrt(var) + eps);"),
    "eps_dropped": ("double rho = 1.0 / sqrt(var + eps);", "double rho = 1.0 / sqrt(var);"),
    "rms_centred": ("if (!is_rms) {", "if (1) {"),
    "mean_not_subtracted": ("double n = (h[c] - mean) * rho;", "double n = h[c] * rho;"),
    "bias_before_weight": ("    if (w) n = n * operand(w, affine_f32, c);\n    if (bias) n = n + operand(bias, affine_f32, c);",
                           "    if (bias) n = n + operand(bias, affine_f32, c);\n    if (w) n = n * operand(w, affine_f32, c);"),
    "frame_index_modulo": ("return b * frames + l / (L / frames);", "return b * frames + l % frames;"),
    "frame_ignores_batch": ("return b * frames + l / (L / frames);", "return l / (L / frames);"),
    "bcast_per_batch": ("case ORC_BCAST: return 0;", "case ORC_BCAST: return b;"),
    "ties_away_from_zero": ("double r = rint(a / q) * q;", "double r = round(a / q) * q;"),
    "round_toward_zero": ("double r = rint(a / q) * q;", "double r = trunc(a / q) * q;"),
    "no_subnormal_quantum": ("if (e < -126) e = -126;", ""),
    "flush_subnormals": ("if (a == 0.0) return sign;", "if (a < 0x1.0p-126) return sign;"),
    "fp8_scale_480": ("float s = (float)(amax / 448.0);", "float s = (float)(amax / 480.0);"),
    "fp8_not_scaled": ("orc_f64_to_e4m3(t[c] / (double)s)", "orc_f64_to_e4m3(t[c])"),
    "e4m3_ties_away": ("double r = isinf(a) ? 512.0 : rint(a / q) * q;",
                       "double r = isinf(a) ? 512.0 : round(a / q) * q;"),
    "e4m3_exponent_bias": ("int exp_field = (er - 1) + 7;", "int exp_field = (er - 1) + 8;"),
    "e4m3_no_saturation": ("if (r > 448.0) r = 448.0;", ""),
    "affine_f32_read_as_bf16": ("return f32 ? (double)((const float*)p)[c] : orc_bf16_to_f64(((const uint16_t*)p)[c]);",
                                "return orc_bf16_to_f64(((const uint16_t*)p)[c]);"),
    "y_f32_via_bf16": ("((float*)y_row)[c] = (float)t[c];",
                       "((float*)y_row)[c] = (float)orc_bf16_to_f64(orc_f64_to_bf16(t[c]));"),
    "gate_row_from_ss_layout": ("const uint16_t* g_row = gate ? gate + orc_mod_row(gate_kind, gate_frames, r, L) * D : NULL;",
                                "const uint16_t* g_row = gate ? gate + orc_mod_row(ss_kind, ss_frames, r, L) * D : NULL;"),
}


def _run_pins(o):
    failed = []
    checks = list(pins.FAST_PINS) + [
        lambda o: pins.pin_residual_vs_torch(o, n_res=16, n_gate=6),
        lambda o: pins.pin_round_f32_vs_torch(o, stride=65521, threads=4),
        lambda o: pins.pin_bruteforce_d8(o, stride=97, threads=4),
        lambda o: pins.pin_e4m3_vs_torch(o, stride=4099, threads=4),
    ]
    for pin in checks:
        try:
            pin(o)
        except AssertionError:
            failed.append(getattr(pin, "__name__", "lambda"))
        except ValueError:
            failed.append(getattr(pin, "__name__", "lambda"))
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle.SRC).read()
    before, after = MUTANTS[name]
    assert before in src, "mutation site missing: %s" % name
    mutated = src.replace(before, after, 1)
    csrc = tmp_path / "oracle.c"
    csrc.write_text(mutated)
    (tmp_path / "oracle.h").write_text(open(os.path.join(os.path.dirname(oracle.SRC),
                                                         "oracle.h")).read())
    lib = oracle.build(str(csrc), str(tmp_path / "liboracle_mut.so"))
    failed = _run_pins(oracle.Oracle(lib))
    assert failed, "no pin caught mutant %s" % name


def test_unmutated_copy_passes_all(tmp_path):
    """The same harness accepts the real oracle (so a caught mutant is the mutation)."""
    lib = oracle.build(oracle.SRC, str(tmp_path / "liboracle_copy.so"))
    assert _run_pins(oracle.Oracle(lib)) == []
