"""Plant mistakes in copies of the oracle and check that the pins catch each.

Every mutant is a text edit of ``oracle/lse_oracle.c`` compiled into a
temporary directory; the real oracle is never touched. A mutant that passes
every pin would mean the pins could not tell that mistake from the truth.
"""
import shutil

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "no_max_shift": ("s += exp(load_elem(x, dtype, start + j) - m);",
                     "s += exp(load_elem(x, dtype, start + j));"),
    "minus_log": ("return m + log(s);", "return m - log(s);"),
    "dropped_max": ("return m + log(s);", "return log(s);"),
    "dropped_first_term": ("for (j = 0; j < cols; ++j)\n        s +=",
                           "for (j = 1; j < cols; ++j)\n        s +="),
    "dropped_last_term": ("for (j = 0; j < cols; ++j)\n        s +=",
                          "for (j = 0; j + 1 < cols; ++j)\n        s +="),
    "max_skips_first": ("for (j = 0; j < cols; ++j) {", "for (j = 1; j < cols; ++j) {"),
    "min_not_max": ("if (v > m)", "if (v < m)"),
    "bf16_shift_15": ("w = (uint32_t)h << 16;", "w = (uint32_t)h << 15;"),
    "bf16_low_half": ("w = (uint32_t)h << 16;", "w = (uint32_t)h;"),
    "f16_bias_14": ("v = ldexp((double)(1024 + frac), e - 25);",
                    "v = ldexp((double)(1024 + frac), e - 24);"),
    "f16_no_implicit_one": ("v = ldexp((double)(1024 + frac), e - 25);",
                            "v = ldexp((double)frac, e - 25);"),
    "f16_subnormal_scale": ("v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    "f16_sign_dropped": ("return sign ? -v : v;", "return (sign && 0) ? -v : v;"),
    "f16_decoded_as_bf16": ("} else if (dtype == ORACLE_F16) {", "} else if (dtype == -1) {"),
    "f32_wrong_width": ("(const char *)x + 4 * index", "(const char *)x + 2 * index"),
    "row_start_uses_cols": ("jb->out[r] = lse_one_row(jb->x, jb->dtype, r * jb->row_stride",
                            "jb->out[r] = lse_one_row(jb->x, jb->dtype, r * jb->cols"),
    "logprob_row_start_uses_cols": ("token_logprob_one_row(jb->x, jb->dtype, r * jb->row_stride",
                                    "token_logprob_one_row(jb->x, jb->dtype, r * jb->cols"),
    "logprob_sign": ("return load_elem(x, dtype, start + t) - lse_one_row(",
                     "return lse_one_row(x, dtype, start, cols) - load_elem(x, dtype, start + t) + 0 * lse_one_row("),
    "logprob_next_column": ("return load_elem(x, dtype, start + t) - lse_one_row(",
                            "return load_elem(x, dtype, start + (t + 1) % cols) - lse_one_row("),
    "logprob_drops_lse": ("return load_elem(x, dtype, start + t) - lse_one_row(x, dtype, start, cols);",
                          "return load_elem(x, dtype, start + t);"),
    "logprob_drops_element": ("return load_elem(x, dtype, start + t) - lse_one_row(x, dtype, start, cols);",
                              "return -lse_one_row(x, dtype, start, cols);"),
    "logprob_out_of_range_zero": ("if (t < 0 || t >= cols)\n        return NAN;",
                                  "if (t < 0 || t >= cols)\n        return 0.0;"),
    "grad_sign": ("out[j] = grad_out * exp(load_elem(x, dtype, start + j) - lse);",
                  "out[j] = grad_out * exp(lse - load_elem(x, dtype, start + j));"),
    "grad_drops_grad_out": ("out[j] = grad_out * exp(load_elem(x, dtype, start + j) - lse);",
                            "out[j] = exp(load_elem(x, dtype, start + j) - lse);"),
    "grad_exp2": ("out[j] = grad_out * exp(load_elem(", "out[j] = grad_out * exp2(load_elem("),
    "grad_wrong_row_lse": ("(double)jb->lse[r], (double)jb->grad_out[r],",
                           "(double)jb->lse[r == jb->row_begin ? r : r - 1], (double)jb->grad_out[r],"),
    "grad_column_shift": ("exp(load_elem(x, dtype, start + j) - lse)",
                          "exp(load_elem(x, dtype, start + (j + 1) % cols) - lse)"),
    "grad_every_row_into_row0": ("jb->out + r * jb->cols);", "jb->out);"),
    "logprob_wrong_row_target": ("jb->targets[r]);", "jb->targets[r == jb->row_begin ? r : r - 1]);"),
    "nan_not_checked_with_inf": ("if (m == INFINITY)\n        return INFINITY;",
                                 "if (m == INFINITY && 0)\n        return INFINITY;"),
    "nan_check_removed": ("if (isnan(v))\n            return NAN;", ""),
    "neg_inf_guard_removed": ("if (m == -INFINITY)\n        return -INFINITY;", ""),
    "rows_per_thread_floor": ("per = (rows + nthreads - 1) / nthreads;",
                              "per = rows / nthreads;"),
    "log2_not_ln": ("return m + log(s);", "return m + log2(s);"),
    "exp2_not_exp": ("s += exp(load_elem", "s += exp2(load_elem"),
    "tokgrad_sign": ("out[k] = valid ? g * ((k == t ? 1.0 : 0.0) - p) : NAN;",
                     "out[k] = valid ? g * ((k == t ? 1.0 : 0.0) + p) : NAN;"),
    "tokgrad_onehot_next_column": ("(k == t ? 1.0 : 0.0)", "(k == (t + 1) % cols ? 1.0 : 0.0)"),
    "tokgrad_onehot_not_scaled": ("g * ((k == t ? 1.0 : 0.0) - p)", "((k == t ? 1.0 : 0.0) - g * p)"),
    "tokgrad_invalid_target_zero": ("out[k] = valid ? g * ((k == t ? 1.0 : 0.0) - p) : NAN;",
                                    "out[k] = valid ? g * ((k == t ? 1.0 : 0.0) - p) : 0.0;"),
    "tokgrad_row_start_uses_cols": ("token_grad_one_row(jb->x, jb->dtype, r * jb->row_stride",
                                    "token_grad_one_row(jb->x, jb->dtype, r * jb->cols"),
    "tokgrad_wrong_row_lse": ("jb->lse[r], jb->grad_out[r], &jb->out[r * jb->cols]);",
                              "jb->lse[r == jb->row_begin ? r : r - 1], jb->grad_out[r], &jb->out[r * jb->cols]);"),
}


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = oracle.SOURCE.read_text()
    assert src.count(old) == 1, f"mutation site for {name} not unique in the oracle source"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(old, new))
    lib = oracle.build(mutant_src, tmp_path / "libmutant.so")
    orc = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.CHEAP_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
            break
    assert caught, f"mutant {name} passed every pin"
