"""Planted mistakes in copies of the C oracle must fail its pins.

Each case below edits lema_oracle.c the way a plausible misreading or slip
would (a dropped term, a wrong sign or coefficient, a different rounding, an
index off by one), builds the edited copy with the oracle's own gcc flags into
a temporary directory, binds it in place of the real library, and runs the
pins of tests/test_oracle_pins.py and tests/test_oracle_q8_pins.py against
it.  Only the copies are altered; the real oracle is restored after each case.

Every mistake must be caught by a pin grounded outside the oracle (a closed
form, exact rational arithmetic, torch.optim.AdamW, a hand-computed example,
an invariant); the bit-exact comparisons with the independent Python
implementation are not counted here.
"""
from __future__ import annotations

import contextlib
import ctypes
import subprocess

import pytest

import oracle
import test_oracle_pins as P
import test_oracle_q8_pins as Q

# pins with a reference outside the oracle
MATH_PINS = [
    ("constants exact t=1", lambda: P.test_constants_against_exact_arithmetic(1)),
    ("constants exact t=12345", lambda: P.test_constants_against_exact_arithmetic(12345)),
    ("constants known values", P.test_constants_known_values),
    ("rne16 textbook", P.test_rne16_textbook_on_boundaries),
    ("rne16 specials", P.test_rne16_special_values),
    ("zero gradient t=1", lambda: P.test_zero_gradient_fresh_state(1)),
    ("zero gradient t=100", lambda: P.test_zero_gradient_fresh_state(100)),
    ("zero lr", P.test_zero_lr_keeps_weights),
    ("zero betas", lambda: P.test_zero_betas_sign_sgd(7)),
    ("eps placement", lambda: P.test_step1_eps_placement(1e-8)),
    ("step-1 closed form", P.test_step1_closed_form_every_element),
    ("torch AdamW t=10", lambda: P.test_against_torch_adamw(10)),
    ("torch AdamW t=100", lambda: P.test_against_torch_adamw(100)),
    ("accumulation exact sums", P.test_accumulate_exact_sums),
    ("accumulation specials", P.test_accumulate_overwrite_keeps_negative_zero_and_specials),
    ("delta reconstructs", P.test_delta_reconstructs_master),
    ("delta zero", P.test_delta_zero_when_master_equals_base),
    ("nan and inf", P.test_nan_and_inf_propagate),
    ("merge reproduces weight", P.test_merge_delta_reproduces_step_weight),
    ("q8 worked example", Q.test_worked_example_power_of_two_scales),
    ("q8 scale exact", Q.test_scale_is_absmax_over_127_exactly_rounded),
    ("q8 codes exact", Q.test_codes_are_nearest_integers_of_the_exact_quotient),
    ("q8 row mapping", Q.test_rows_map_to_their_own_scales_with_ragged_tail),
    ("q8 special rows", Q.test_special_rows),
    ("q8 subnormal scale", Q.test_subnormal_scale_keeps_codes_in_range),
    ("q8 step on grid moments", lambda: Q.test_q8_step_is_the_fp32_step_on_dequantized_state("bf16")),
    ("q8 step, int8 gradient", lambda: Q.test_q8_step_is_the_fp32_step_on_dequantized_state("q8")),
    ("q8 fresh step", Q.test_q8_step_fresh_state_first_step_closed_form),
    ("q8 accumulation on grid", Q.test_q8_accumulation_exact_on_grid),
]

# (name, [(text in lema_oracle.c, replacement)])
MUTANTS = [
    ("no_weight_decay",
     [("float w_decayed = master[i] * decay;", "float w_decayed = master[i];")]),
    ("weight_decay_after_update",
     [("float w_new = w_decayed - update;", "float w_new = (master[i] - update) * decay;")]),
    ("eps_inside_root",
     [("float denom = root_hat + eps;", "float denom = sqrtf(root_hat * root_hat + eps);")]),
    ("second_moment_with_beta1",
     [("float v_old_part = b2 * v[i];", "float v_old_part = b1 * v[i];")]),
    ("first_moment_with_1_minus_beta2",
     [("float m_new_part = one_minus_b1 * g;", "float m_new_part = one_minus_b2 * g;")]),
    ("second_moment_of_abs_g",
     [("float g_squared = g * g;", "float g_squared = fabsf(g);")]),
    ("update_sign_flipped",
     [("float w_new = w_decayed - update;", "float w_new = w_decayed + update;")]),
    ("update_fused_multiply_add",
     [("float w_new = w_decayed - update;", "float w_new = fmaf(-step_size, ratio, w_decayed);")]),
    ("no_bias_correction_1",
     [("out[6] = (float)(lr / bc1);", "out[6] = (float)lr;")]),
    ("bias_correction_2_without_root",
     [("out[7] = (float)(1.0 / sqrt(bc2));", "out[7] = (float)(1.0 / bc2);")]),
    ("step_count_off_by_one",
     [("double bc1 = 1.0 - power_by_squaring(beta1, t);",
       "double bc1 = 1.0 - power_by_squaring(beta1, t + 1);")]),
    ("decay_without_weight_decay_factor",
     [("out[5] = (float)(1.0 - lr * weight_decay);", "out[5] = (float)(1.0 - lr);")]),
    ("bf16_truncation",
     [("if (dropped > 0x8000u)", "if (dropped > 0xFFFFu)"),
      ("else if (dropped == 0x8000u && (kept & 1u))", "else if (0)")]),
    ("bf16_ties_away_from_zero",
     [("else if (dropped == 0x8000u && (kept & 1u))", "else if (dropped == 0x8000u)")]),
    ("accumulation_overwrite_adds",
     [("            acc[i] = gi;", "            acc[i] = acc[i] + gi;")]),
    ("delta_against_decayed_weight",
     [("delta[i] = w_new - oracle_bf16_to_f32(orig[i]);", "delta[i] = w_new - w_decayed;")]),
    ("merge_rounds_delta_first",
     [("float sum = oracle_bf16_to_f32(base[i]) + delta[i];",
       "float sum = oracle_bf16_to_f32(base[i]) + oracle_bf16_to_f32(oracle_rne16(delta[i]));")]),
    ("int8_half_away_from_zero",
     [("float k = rintf(r);", "float k = roundf(r);")]),
    ("int8_reciprocal_scale",
     [("float r = x / scale;", "float r = x * (1.0f / scale);")]),
    ("int8_divisor_128",
     [("float s = row_absmax(x + lo, len) / 127.0f;",
       "float s = row_absmax(x + lo, len) / 128.0f;")]),
    ("int8_clamp_at_128",
     [("if (k > 127.0f)\n        k = 127.0f;", "if (k > 128.0f)\n        k = 128.0f;")]),
    ("int8_row_index_shifted",
     [("x[i] = (float)q[i] * scale[i / row_len];",
       "x[i] = (float)q[i] * scale[(i > 0 ? i - 1 : 0) / row_len];")]),
    ("int8_nan_ignored",
     [("            saw_nan = 1;", "            saw_nan = 0;")]),
]


@pytest.fixture(scope="module")
def source():
    with open(oracle._SRC) as f:
        return f.read()


def build_copy(source: str, edits, directory, name: str) -> str:
    text = source
    for old, new in edits:
        assert text.count(old) == 1, f"{name}: edit target not found once: {old!r}"
        text = text.replace(old, new)
    c_path = directory / f"{name}.c"
    so_path = directory / f"lib{name}.so"
    c_path.write_text(text)
    subprocess.run(["gcc", *oracle.GCC_FLAGS, "-o", str(so_path), str(c_path), "-lm"],
                   check=True, capture_output=True)
    return str(so_path)


@contextlib.contextmanager
def bound(so_path: str):
    saved = oracle._load()
    oracle._lib = oracle.bind(ctypes.CDLL(so_path))
    try:
        yield
    finally:
        oracle._lib = saved


def first_failure(pins):
    for label, fn in pins:
        try:
            fn()
        except Exception:           # an assertion, or a crash on bad output
            return label
    return None


def test_unaltered_copy_passes_every_pin(source, tmp_path):
    """The harness itself: the oracle rebuilt from unaltered source through
    the same path passes every pin, so a failure below is the planted
    mistake's doing."""
    with bound(build_copy(source, [], tmp_path, "unaltered")):
        for label, fn in MATH_PINS:
            fn()


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(source, tmp_path, name, edits):
    with bound(build_copy(source, edits, tmp_path, name)):
        caught = first_failure(MATH_PINS)
    assert caught is not None, f"{name}: no pin grounded outside the oracle fails"
    print(f"{name}: caught by {caught}")


# Mistakes in the Python composition of the int8 functions (oracle/__init__.py):
# (name, [(text, replacement)])
PY_MUTANTS = [
    ("int8_step_skips_requantization",
     [("            arr[0][...] = q\n            arr[1][...] = s", "            pass")]),
    ("int8_overwrite_adds_to_old_accumulator",
     [("        acc = np.zeros(n, dtype=np.float32)",
       "        acc = dequantize_rows(acc_q, acc_scale, row_len)"),
      ("    grad_accum(acc, grad_bf16, overwrite)", "    grad_accum(acc, grad_bf16, False)")]),
    ("int8_gradient_not_dequantized",
     [("        grad = dequantize_rows(grad[0], grad[1], row_len)",
       "        grad = grad[0].astype(np.float32)")]),
]


@contextlib.contextmanager
def python_copy(edits, directory, name):
    """A copy of the oracle package's module with `edits`, bound to the real
    library, put in place of `oracle` inside the pin modules."""
    import importlib.util
    with open(oracle.__file__) as f:
        text = f.read()
    for old, new in edits:
        assert text.count(old) == 1, f"{name}: edit target not found once: {old!r}"
        text = text.replace(old, new)
    path = directory / f"oracle_{name}.py"
    path.write_text(text)
    spec = importlib.util.spec_from_file_location(f"oracle_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod._lib = oracle._load()
    saved = P.oracle, Q.oracle
    P.oracle = Q.oracle = mod
    try:
        yield
    finally:
        P.oracle, Q.oracle = saved


def test_unaltered_python_copy_passes_every_pin(tmp_path):
    with python_copy([], tmp_path, "unaltered"):
        for label, fn in MATH_PINS:
            fn()


@pytest.mark.parametrize("name,edits", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_planted_composition_mistake_fails_a_pin(tmp_path, name, edits):
    with python_copy(edits, tmp_path, name):
        caught = first_failure(MATH_PINS)
    assert caught is not None, f"{name}: no pin grounded outside the oracle fails"
    print(f"{name}: caught by {caught}")
