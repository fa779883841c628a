"""Planted mistakes: each mutant is a copy of the oracle's C source with one
plausible slip (a flipped sign, a wrong index, a dropped term, a transposed
operand, a wrong rounding rule).  It is compiled on the CPU and loaded in
place of the oracle; at least one pin from test_oracle_pins must then fail.
This shows the pins would notice such a slip in the real oracle."""
from __future__ import annotations

import ctypes
import os
import shutil
import subprocess
import tempfile

import pytest

import oracle
from tests import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "mla_oracle.c")

# (name, text in the source, replacement) -- each text occurs exactly once
MUTANTS = [
    ("rope_sign", "y[i0] = ac - bs;", "y[i0] = ac + bs;"),
    ("rope_dropped_term", "y[i1] = bc + as;", "y[i1] = bc;"),
    ("rope_neox_pair_index", "*i1 = p + HALF; }", "*i1 = p + HALF - 1; }"),
    ("rope_gptj_pair_swapped", "*i0 = 2 * p; *i1 = 2 * p + 1; }", "*i0 = 2 * p + 1; *i1 = 2 * p; }"),
    ("rope_cos_sin_swapped", "float a = x[i0], b = x[i1], c = cos_row[p], s = sin_row[p];",
     "float a = x[i0], b = x[i1], c = sin_row[p], s = cos_row[p];"),
    ("table_bf16_read_as_fp16", "c[p] = oracle_bf16_to_f32(t[p]);", "c[p] = oracle_fp16_to_f32(t[p]);"),
    ("q_rotated_at_position_zero",
     "q_pe + (size_t)r * PE, rope, gptj, trow,", "q_pe + (size_t)r * PE, rope, gptj, table,"),
    ("k_pe_not_rotated", "k_pe + (size_t)t * PE, rope, gptj", "k_pe + (size_t)t * PE, 0, gptj"),
    ("bf16_truncates", "if (lo > 0x8000u || (lo == 0x8000u && (hi & 1u)))", "if (0)"),
    ("bf16_ties_away", "(lo == 0x8000u && (hi & 1u))", "(lo == 0x8000u)"),
    ("fp16_decode_bias", "ldexp(1.0 + m / 1024.0, e - 15)", "ldexp(1.0 + m / 1024.0, e - 16)"),
    ("fp16_encode_bias", "(uint16_t)((ue + 15) << 10)", "(uint16_t)((ue + 16) << 10)"),
    ("fp16_overflow_threshold", "if (a >= 65520.0) return", "if (a >= 131072.0) return"),
    ("fp16_subnormal_step", "round_half_even(a * 16777216.0)", "round_half_even(a * 8388608.0)"),
    ("fp16_activations_read_as_bf16", "return fp16 ? oracle_fp16_to_f32(v) : oracle_bf16_to_f32(v);",
     "return oracle_bf16_to_f32(v);"),
    ("e4m3_ties_up", "return (fmod(f, 2.0) == 0.0) ? f : f + 1.0;", "return f + 1.0;"),
    ("e4m3_no_saturation", "if (a >= 448.0) return (uint8_t)(sign | 0x7E);",
     "if (a >= 480.0) return (uint8_t)(sign | 0x7F);"),
    ("e4m3_bias", "int be = ue + 7;", "int be = ue + 8;"),
    ("e4m3_subnormal_step", "round_half_even(a * 512.0)", "round_half_even(a * 256.0)"),
    ("quant_by_scale_not_inverse", "float qi = q_fp8 ? 1.0f / q_scale : 1.0f;",
     "float qi = q_fp8 ? q_scale : 1.0f;"),
    ("scatter_by_token", "write_row(cache + (size_t)s * kv_row_bytes", "write_row(cache + (size_t)t * kv_row_bytes"),
    ("slot_zero_skipped", "if (s < 0 || s >= num_slots) continue;", "if (s <= 0 || s >= num_slots) continue;"),
    ("q_rows_transposed", "int64_t r = t * H + h;", "int64_t r = h * T + t;"),
    ("rope_f64_sign", "y[i0] = a * c - b * s;", "y[i0] = a * c + b * s;"),
    ("rope_f64_dropped_term", "y[i1] = b * c + a * s;", "y[i1] = b * c;"),
    ("uk_weight_head_ignored", "w_uk_t + ((size_t)h * NOPE + n) * 128;", "w_uk_t + ((size_t)n) * 128;"),
    ("uk_weight_read_untransposed", "(double)elem_to_f32(w[k], fp16);",
     "(double)elem_to_f32(w_uk_t[((size_t)h * 128 + k) * NOPE + n], fp16);"),
    ("uk_last_k_dropped", "for (int k = 0; k < 128; ++k) {\n                    const double prod",
     "for (int k = 0; k < 127; ++k) {\n                    const double prod"),
    ("uk_query_head_shifted", "q_nope + ((size_t)t * H + h) * 128;", "q_nope + ((size_t)t * H + (h + 1) % H) * 128;"),
    ("uk_magnitude_signed", "acc_abs += fabs(prod);", "acc_abs += prod;"),
    ("uk_fp16_read_as_bf16", "(double)elem_to_f32(q[k], fp16)", "(double)elem_to_f32(q[k], 0)"),
]

CHECKS = [
    P.test_fp16_golden_points,
    P.test_fp16_decode_all_patterns_vs_numpy,
    P.test_fp16_rne_vs_numpy,
    P.test_gptj_rope_golden_rows,
    P.test_gptj_rope_is_complex_rotation_by_position_angle,
    lambda: P.test_oracle_matches_library_composition_variants("bf16", "neox", "bf16", False, False),
    lambda: P.test_oracle_matches_library_composition_variants("fp16", "gptj", "f32", True, False),
    P.test_e4m3_golden_points,
    P.test_e4m3_matches_brute_force_on_all_bf16,
    P.test_bf16_golden_points,
    P.test_bf16_rne_vs_torch,
    P.test_rope_golden_rows,
    P.test_rope_is_complex_rotation_by_position_angle,
    lambda: P.test_page_identity_concat_and_scatter(64),
    lambda: P.test_oracle_matches_library_composition("t64_h16_rope_fp8"),
    lambda: P.test_oracle_matches_library_composition_all_modes((True, False, False)),
    lambda: P.test_oracle_matches_library_composition_all_modes((True, True, False)),
    P.test_out_of_range_slots_leave_cache_untouched,
    lambda: P.test_rope_f64_is_the_complex_product_with_the_table_row(True),
    lambda: P.test_uk_product_matches_library_matmul(False),
    lambda: P.test_uk_product_matches_library_matmul(True),
    P.test_uk_product_unit_rows_select_one_input,
    P.test_uk_product_integers_brute_force,
    P.test_uk_product_magnitude_is_the_absolute_sum,
]


def _caught(lib) -> bool:
    saved = oracle._lib
    oracle._lib = lib
    try:
        for check in CHECKS:
            try:
                check()
            except AssertionError:
                return True
        return False
    finally:
        oracle._lib = saved


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


def _build(src_text: str, d: str, name: str):
    c = os.path.join(d, f"{name}.c")
    so = os.path.join(d, f"lib{name}.so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *oracle.CFLAGS, c, "-o", so, "-lm"], check=True)
    return oracle._configure(ctypes.CDLL(so))


def test_unmutated_copy_passes(workdir):
    with open(SRC) as f:
        text = f.read()
    assert not _caught(_build(text, workdir, "unmutated"))


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(workdir, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    assert _caught(_build(text.replace(old, new), workdir, name)), f"mutant {name} survived the pins"


# ---- the attention oracle (Python): planted slips in a copy of its source ---

from oracle import attention as ATT  # noqa: E402
from tests import test_attention_oracle as AP  # noqa: E402

ATT_SRC = ATT.__file__
ATT_MUTANTS = [
    ("page_index_swapped", "pages = np.asarray(block_table[b])[j // bs]",
     "pages = np.asarray(block_table[b])[j % bs]"),
    ("no_sm_scale", "s = (qd[b] @ rows.T) * sm_scale", "s = (qd[b] @ rows.T)"),
    ("value_from_tail", "out[b] = p @ rows[:, :NOPE]", "out[b] = p @ rows[:, ROW - NOPE:]"),
    ("softmax_over_heads", "p /= p.sum(axis=1, keepdims=True)", "p /= p.sum(axis=0, keepdims=True)"),
    ("e4m3_bias", "np.exp2(e - 7.0)", "np.exp2(e - 8.0)"),
    ("scale_ignored", "return e4m3_decode(x) * float(scale)", "return e4m3_decode(x)"),
    ("last_key_dropped", "j = np.arange(L)", "j = np.arange(max(L - 1, 1))"),
    ("abs_of_sum_not_sum_of_abs", "mag[b] = p @ np.abs(rows[:, :NOPE])",
     "mag[b] = np.abs(p @ rows[:, :NOPE])"),
    ("abs_weights_unnormalised", "mag[b] = p @ np.abs(rows[:, :NOPE])",
     "mag[b] = np.exp(s) @ np.abs(rows[:, :NOPE])"),
]
ATT_CHECKS = [
    AP.test_e4m3_decode_every_code_vs_torch,
    AP.test_single_key_returns_its_value,
    AP.test_two_keys_closed_form,
    AP.test_page_order_invariance,
    lambda: AP.test_matches_library_sdpa(False, False),
    lambda: AP.test_matches_library_sdpa(True, True),
    AP.test_zero_query_averages_values,
    AP.test_weighted_abs_single_key_and_zero_query,
    AP.test_weighted_abs_bounds_and_equality_for_nonnegative_values,
]


def _att_caught(text: str) -> bool:
    import types
    mod = types.ModuleType("attention_mutant")
    exec(compile(text, "attention_mutant.py", "exec"), mod.__dict__)
    saved = (ATT.mla_decode_attention, ATT.e4m3_decode)
    ATT.mla_decode_attention, ATT.e4m3_decode = mod.mla_decode_attention, mod.e4m3_decode
    try:
        for check in ATT_CHECKS:
            try:
                check()
            except (AssertionError, IndexError):   # a wrong index may also fall off the table
                return True
        return False
    finally:
        ATT.mla_decode_attention, ATT.e4m3_decode = saved


def test_attention_unmutated_copy_passes():
    assert not _att_caught(open(ATT_SRC).read())


@pytest.mark.parametrize("name,old,new", ATT_MUTANTS, ids=[m[0] for m in ATT_MUTANTS])
def test_attention_mutant_is_caught(name, old, new):
    text = open(ATT_SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique"
    assert _att_caught(text.replace(old, new)), f"mutant {name} survived the pins"
