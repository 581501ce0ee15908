"""Each pin bites: copies of the oracle with one planted mistake (a dropped
term, a wrong index, swapped halves, a transposed layout, a wrong rounding
point) must fail the pins named for it. Mistakes are planted in oracle.c and
in the oracle's Python side (oracle/__init__.py: the tolerance bound and the
marshalling of the sampled k = 8 form). Runs on the CPU only."""
import importlib.util
import os

import pytest

import oracle
from tests import pins

MUTATIONS = {
    "pack_halves_swapped": (
        "row[16 * kr + 2 * w + 1];\n            P[(((b * rows_rep + r) * K_rep + kr) * R + i) * 8 + w] = lo | (hi << 16);",
        "row[16 * kr + 2 * w + 1];\n            P[(((b * rows_rep + r) * K_rep + kr) * R + i) * 8 + w] = hi | (lo << 16);",
        ["pin_pack_page_recipe", "pin_pack_arange"]),
    "pack_rows_and_k_atoms_transposed": (
        "row[16 * kr + 2 * w + 1];\n            P[(((b * rows_rep + r) * K_rep + kr) * R + i) * 8 + w]",
        "row[16 * kr + 2 * w + 1];\n            P[(((b * rows_rep + r) * R + i) * K_rep + kr) * 8 + w]",
        ["pin_pack_page_recipe", "pin_pack_arange"]),
    "f16_exponent_bias_off_by_one": (
        "expo - 25)", "expo - 24)",
        ["pin_h2f", "pin_page_example", "pin_quarter_closed_form"]),
    "f16_subnormal_scale_wrong": (
        "ldexpf((float)frac, -24)", "ldexpf((float)frac, -25)", ["pin_h2f"]),
    "operand_rows_reversed_in_atom": (
        "* R + row % R) * (ka / 2) + (k % ka) / 2];\n  return oracle_h2f",
        "* R + (R - 1 - row % R)) * (ka / 2) + (k % ka) / 2];\n  return oracle_h2f",
        ["pin_page_example", "pin_quarter_closed_form", "pin_normal_vs_float64"]),
    "c_added_at_every_k16_issue": (
        "acc = acc + a * x;\n  }\n  return acc;",
        "acc = acc + a * x;\n    if (k % 16 == 15 && k + 1 < 16 * K_rep)"
        " acc = acc + (C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c);\n  }\n  return acc;",
        ["pin_quarter_closed_form", "pin_recurrence_chain", "pin_zero_a_and_scalar"]),
    "c_ignored": (
        "float acc = C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c;", "float acc = 0.0f;",
        ["pin_quarter_closed_form", "pin_zero_a_and_scalar", "pin_recurrence_chain"]),
    "accumulator_in_double": (
        "float acc = C ? C[", "double acc = C ? C[",
        ["pin_normal_vs_float64", "pin_recurrence_chain"]),
    "output_atom_transposed": (
        "* N_rep + n / 8) * 16 + m % 16) * 8 + n % 8;",
        "* N_rep + n / 8) * 8 + n % 8) * 16 + m % 16;",
        ["pin_page_example", "pin_quarter_closed_form"]),
    "last_k_atom_dropped": (
        ": c;\n  for (int64_t k = 0; k < ka * K_rep; ++k) {",
        ": c;\n  for (int64_t k = 0; k < ka * K_rep - ka; ++k) {",
        ["pin_page_example", "pin_quarter_closed_form"]),
    "kmajor_k_and_row_strides_swapped": (
        "uint32_t lo = col[(16 * kr + 2 * w) * ld];\n            uint32_t hi = col[(16 * kr + 2 * w + 1) * ld];",
        "uint32_t lo = col[(16 * kr + 2 * w) * ld];\n            uint32_t hi = col[(16 * kr + 2 * w) * ld + 1];",
        ["pin_pack_kmajor"]),
    "scaled_two_roundings": (
        "return fmaf(alpha, acc, t);", "return alpha * acc + t;", ["pin_scaled"]),
    "scaled_beta_ignored": (
        "const float t = beta * cv;", "const float t = cv;", ["pin_scaled"]),
    "k8_word_stride_as_k16": (
        "* R + row % R) * (ka / 2) + (k % ka) / 2];", "* R + row % R) * 8 + (k % ka) / 2];",
        ["pin_k8_layout"]),
    "k8_pack_halves_swapped": (
        "P[(((b * rows_rep + r) * K_rep + kr) * R + i) * 4 + w] = lo | (hi << 16);",
        "P[(((b * rows_rep + r) * K_rep + kr) * R + i) * 4 + w] = hi | (lo << 16);",
        ["pin_k8_layout"]),
    "box_fill_not_zero": (
        "memset(out, 0, (size_t)elem_bytes);", "memset(out, 0x5a, (size_t)elem_bytes);",
        ["pin_box_oob"]),
    "box_repeat_step_ignored": (
        "coords[d] + (int64_t)t * coord_step[d] + j[d]", "coords[d] + j[d]",
        ["pin_box_page_example", "pin_box_oob"]),
    "box_image_repeat_innermost": (
        "img + ((int64_t)t * box_elems + e) * elem_bytes",
        "img + (e * n_repeat + t) * elem_bytes",
        ["pin_box_page_example", "pin_box_oob"]),
    "store_writes_outside": (
        "      if (!inside) continue;\n      const uint8_t* in",
        "      if (!inside) off = 0;\n      const uint8_t* in",
        ["pin_box_store_oob", "pin_box_reduce_order"]),
    "store_repeats_reversed": (
        "const int64_t g = coords[d] + coord_step[d] * (int64_t)t + j[d];",
        "const int64_t g = coords[d] + coord_step[d] * (int64_t)(n_repeat - 1 - t) + j[d];",
        ["pin_box_store_oob", "pin_box_reduce_order"]),
    "reduce_f16_truncates": (
        "const double q = ldexp(1.0, lead - (p - 1)); /* spacing of representable values near x */\n"
        "  const double r = nearbyint(x / q) * q;",
        "const double q = ldexp(1.0, lead - (p - 1)); /* spacing of representable values near x */\n"
        "  const double r = trunc(x / q) * q;",
        ["pin_box_reduce_library_adds"]),
    "reduce_no_overflow_to_inf": (
        "if (fabs(r) > max_finite) return copysign(INFINITY, x);",
        "if (fabs(r) > max_finite) return copysign(max_finite, x);",
        ["pin_box_reduce_library_adds"]),
    "splitk_boundary_rounded_up": (
        "int64_t hi = 32 * ((s + 1) * steps / S);",
        "int64_t hi = 32 * (((s + 1) * steps + S - 1) / S);",
        ["pin_splitk_boundaries_and_order"]),
    "splitk_partials_summed_before_c": (
        '  float d = C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c;\n  for (int64_t s = 0; s < S; ++s) {\n    const int64_t lo = 32 * (s * steps / S);\n    int64_t hi = 32 * ((s + 1) * steps / S);\n    if (hi > K) hi = K;\n    float part = 0.0f;\n    for (int64_t k = lo; k < hi; ++k) {\n      float a = packed_elem(A, b, m, k, 16, M_rep, K_rep, ka, dtype);\n      float x = packed_elem(B, b, n, k, 8, N_rep, K_rep, ka, dtype);\n      part = part + a * x;\n    }\n    d = d + part;\n  }\n  return d;',
        '  float d = 0.0f;\n  for (int64_t s = 0; s < S; ++s) {\n    const int64_t lo = 32 * (s * steps / S);\n    int64_t hi = 32 * ((s + 1) * steps / S);\n    if (hi > K) hi = K;\n    float part = 0.0f;\n    for (int64_t k = lo; k < hi; ++k) {\n      float a = packed_elem(A, b, m, k, 16, M_rep, K_rep, ka, dtype);\n      float x = packed_elem(B, b, n, k, 8, N_rep, K_rep, ka, dtype);\n      part = part + a * x;\n    }\n    d = d + part;\n  }\n  return S ? d + (C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c) : (C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c);',
        ["pin_splitk_boundaries_and_order"]),
    "splitk_c_ignored": (
        "  float d = C ? C[acc_offset(b, m, n, M_rep, N_rep)] : c;\n  for (int64_t s = 0;",
        "  float d = 0.0f;\n  for (int64_t s = 0;",
        ["pin_splitk_exact_and_degenerate", "pin_splitk_boundaries_and_order",
         "pin_splitk_normal_and_layouts"]),
    "splitk_last_range_dropped": (
        "  for (int64_t s = 0; s < S; ++s) {\n    const int64_t lo",
        "  for (int64_t s = 0; s + 1 < S; ++s) {\n    const int64_t lo",
        ["pin_splitk_exact_and_degenerate", "pin_splitk_normal_and_layouts"]),
}


# Planted in oracle/__init__.py; each copy is loaded as a module of its own
# and drives the unmodified liboracle.so.
PY_MUTATIONS = {
    "abs_mask_keeps_low_half_sign": (
        "& np.uint32(0x7FFF7FFF)", "& np.uint32(0x7FFFFFFF)", ["pin_bound"]),
    "abs_mask_keeps_high_half_sign": (
        "& np.uint32(0x7FFF7FFF)", "& np.uint32(0xFFFF7FFF)", ["pin_bound"]),
    "bound_c_tensor_not_absolute": (
        "Ca = None if C is None else np.abs(C)", "Ca = C", ["pin_bound"]),
    "bound_scalar_c_not_absolute": (
        "return self.mma(Aa, Ba, Ca, abs(float(c)), dtype)\n"
        "        return self.mma_sampled(Aa, Ba, Ca, abs(float(c)), dtype, idx)",
        "return self.mma(Aa, Ba, Ca, float(c), dtype)\n"
        "        return self.mma_sampled(Aa, Ba, Ca, float(c), dtype, idx)",
        ["pin_bound"]),
    "bound_sampled_ignores_c": (
        "return self.mma_sampled(Aa, Ba, Ca, abs(float(c)), dtype, idx)",
        "return self.mma_sampled(Aa, Ba, None, abs(float(c)), dtype, idx)",
        ["pin_bound"]),
    "k8_sampled_read_as_k16_layout": (
        "_ptr(C), float(c), batch, M_rep, N_rep, K_rep, 8,",
        "_ptr(C), float(c), batch, M_rep, N_rep, K_rep // 2, 16,",
        ["pin_k8_sampled_matches_full"]),
    "k8_sampled_c_dropped": (
        "_ptr(C), float(c), batch, M_rep, N_rep, K_rep, 8,",
        "None, float(c), batch, M_rep, N_rep, K_rep, 8,",
        ["pin_k8_sampled_matches_full"]),
}


def _run_pins(o, expected):
    failed = []
    for pin in expected:
        try:
            pins.ALL_PINS[pin](o)
        except (AssertionError, ValueError):
            failed.append(pin)
    return failed


@pytest.mark.parametrize("name", sorted(PY_MUTATIONS))
def test_python_side_mutation_is_caught(name, tmp_path):
    old, new, expected = PY_MUTATIONS[name]
    path = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "__init__.py")
    src = open(path).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    mod_path = os.path.join(tmp_path, "mutated_oracle.py")
    with open(mod_path, "w") as f:
        f.write(src.replace(old, new))
    spec = importlib.util.spec_from_file_location(f"mutated_oracle_{name}", mod_path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    o = mod.Oracle(oracle.build(force=False))
    failed = _run_pins(o, expected)
    assert failed == expected, f"{name}: only {failed} of {expected} caught it"
    # the unmutated pins pass on the same library
    assert _run_pins(oracle.default(), expected) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new, expected = MUTATIONS[name]
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
    path = oracle.build_variant(src.replace(old, new), os.path.join(tmp_path, f"lib_{name}.so"))
    o = oracle.Oracle(path)
    failed = []
    for pin in expected:
        try:
            pins.ALL_PINS[pin](o)
        except (AssertionError, ValueError):
            failed.append(pin)
    assert failed == expected, f"{name}: only {failed} of {expected} caught it"
