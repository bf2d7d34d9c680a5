"""The CPU oracle against its pins (library routines, closed forms, brute force,
invariants).  See pins.py for what each pin fixes and where it comes from."""
import pytest

import pins


def test_round_f32_exhaustive_vs_torch(orc):
    pins.pin_round_f32_vs_torch(orc)


def test_round_f64_nearest_table(orc):
    pins.pin_round_f64(orc)


def test_residual_all_bf16_x_vs_torch(orc):
    pins.pin_residual_vs_torch(orc)


def test_residual_gate_zero_is_identity(orc):
    pins.pin_residual_gate_zero(orc)


def test_residual_one_rounding_below_the_normal_range(orc):
    pins.pin_residual_one_rounding(orc)


def test_closed_forms(orc):
    pins.pin_closed_forms(orc)


def test_modulation_special_cases(orc):
    pins.pin_modulation(orc)


def test_torch_layer_norm_rms_norm_float64(orc):
    pins.pin_torch_norms(orc)


def test_layout_addressing_and_equivalences(orc):
    pins.pin_layouts(orc)


def test_fused_normalises_its_residual_output(orc):
    pins.pin_fused_is_nss_of_residual(orc)


def test_scale_invariance_eps0(orc):
    pins.pin_scale_invariance(orc)


def test_bruteforce_d8_dyadic_exhaustive(orc):
    pins.pin_bruteforce_d8(orc)


def test_random_rows_extended_precision(orc):
    pins.pin_random_rows_ld(orc)


def test_norm_invariants(orc):
    pins.pin_invariants(orc)


def test_e4m3_vs_torch(orc):
    pins.pin_e4m3_vs_torch(orc)


def test_affine_f32(orc):
    pins.pin_affine_f32(orc)


def test_y_f32(orc):
    pins.pin_y_f32(orc)


def test_fp8_rows(orc):
    pins.pin_fp8_rows(orc)
