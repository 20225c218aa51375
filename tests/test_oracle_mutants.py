"""The pins are sharp enough: each planted mistake in a copy of the oracle fails at least one.

Every mutant is a one-line edit of the oracle's C source of the kind a careless port would
make (a dropped term, a wrong sign, a swapped operand or index).  It is built into a temporary
library, every oracle call is routed to it, and the pin tests of ``test_oracle`` are run
against it; at least one must fail.  Mutants are chosen so they stay in bounds (none can make
the oracle read outside its arrays).
"""

import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "longattn_oracle.c")

MUTANTS = {
    "window_extents_swapped": ("int64_t t_lo = -p->win_left, t_hi = p->win_right;",
                               "int64_t t_lo = -p->win_right, t_hi = p->win_left;"),
    "dilation_ignored": ("int64_t dil = p->dilation ? p->dilation[h] : 1;", "int64_t dil = 1;"),
    "band_right_edge_short": ("int64_t t_max_in = floor_div(p->n - 1 - i, dil);",
                              "int64_t t_max_in = floor_div(p->n - 2 - i, dil);"),
    "padding_ignored": ("  if (p->key_pad && p->key_pad[b * p->n + j]) return;", ""),
    "global_rows_not_full": ("if (is_global && is_global[b * p->n + i]) {", "if (0) {"),
    "global_columns_dropped": (
        "for (int64_t c = 0; c < p->n_global; ++c) add_key(w, p, b, p->global_idx[b * p->n_global + c]);",
        ""),
    "softmax_sign_flipped": ("double wt = exp(w.s[t] - m);", "double wt = exp(m - w.s[t]);"),
    "scale_dropped": ("w.s[t] = scale * dot;", "w.s[t] = dot;"),
    "values_read_from_keys": ("const double* vj = vb + (int64_t)w.keys[t] * p->d;",
                              "const double* vj = kb + (int64_t)w.keys[t] * p->d;"),
    "lse_without_log": ("if (lse) lse[r] = m + log(l);", "if (lse) lse[r] = m + l;"),
    "no_normalisation": ("for (int64_t c = 0; c < p->d; ++c) oi[c] /= l;", ""),
    "empty_row_lse_zero": ("if (lse) lse[r] = -INFINITY;", "if (lse) lse[r] = 0.0;"),
    "layout_block_of_key_not_query": (
        "const int32_t* row = p->layout + (h * nb + i / p->block) * p->max_kb;",
        "const int32_t* row = p->layout + (h * nb + (i % nb)) * p->max_kb;"),
    "layout_block_width_off": (
        "for (int64_t j = (int64_t)row[s] * p->block; j < ((int64_t)row[s] + 1) * p->block; ++j)",
        "for (int64_t j = (int64_t)row[s] * p->block; j < ((int64_t)row[s] + 1) * p->block - 1; ++j)"),
    "query_row_of_other_head": ("const double* qi = q + r * p->d;",
                                "const double* qi = q + (r % p->n) * p->d;"),
}

PINS = [
    lambda: [pins.test_oracle_matches_dense_brute_force(c) for c in pins.CASES],
    lambda: pins.test_window_covering_sequence_is_full_attention(37, 8),
    lambda: pins.test_causal_window_covering_sequence_is_causal_attention(50),
    pins.test_layout_listing_every_block_is_full_attention,
    pins.test_softmax_rows_sum_to_one,
    pins.test_keys_outside_the_set_contribute_exactly_zero,
    pins.test_bigbird_worked_window_example,
    pins.test_window_zero_returns_v_exactly,
    pins.test_zero_keys_give_the_mean_of_values,
    lambda: pins.test_band_count_closed_form(100, 7, 2),
    lambda: pins.test_dilated_row_counts(101, 3, 4, 9),
    pins.test_empty_rows_give_zero_output_and_minus_infinity_lse,
    pins.test_bigbird_global_blocks_as_layout_or_as_global_tokens,
    pins.test_global_rows_attend_every_unpadded_key_and_padding_wins,
]


# Planted mistakes in the backward pass, caught by the backward pins.
from tests import test_oracle_backward as bpins  # noqa: E402

BWD_MUTANTS = {
    "bwd_drow_dropped": ("const double ds = w.s[t] * (dp[t] - drow);",
                         "const double ds = w.s[t] * dp[t];"),
    "bwd_ds_sign_flipped": ("const double ds = w.s[t] * (dp[t] - drow);",
                            "const double ds = w.s[t] * (drow - dp[t]);"),
    "bwd_dq_scale_dropped": ("dqi[c] += scale * ds * kj[c];", "dqi[c] += ds * kj[c];"),
    "bwd_dk_uses_key": ("dkb[j * d + c] += scale * ds * qi[c];",
                        "dkb[j * d + c] += scale * ds * kj[c];"),
    "bwd_dv_uses_ds": ("dvb[j * d + c] += w.s[t] * doi[c];", "dvb[j * d + c] += ds * doi[c];"),
    "bwd_dp_against_keys": ("const double* vj = vb + (int64_t)w.keys[t] * d;\n          double dot = 0.0;\n          for (int64_t c = 0; c < d; ++c) dot += doi[c] * vj[c];",
                            "const double* vj = kb + (int64_t)w.keys[t] * d;\n          double dot = 0.0;\n          for (int64_t c = 0; c < d; ++c) dot += doi[c] * vj[c];"),
    "bwd_unnormalised_weights": ("w.s[t] = exp(w.s[t] - lse); /* P_j from here on */",
                                 "w.s[t] = exp(w.s[t] - m); /* P_j from here on */"),
    "bwd_dq_of_other_head": ("double* dqi = dq + r * d;", "double* dqi = dq + (r % n) * d;"),
}

BWD_PINS = [
    lambda: [bpins.test_backward_matches_finite_differences_of_the_forward(c) for c in bpins.SMALL],
    lambda: [bpins.test_backward_matches_autograd_of_dense_masked_attention(c)
             for c in bpins.BRUTE],
    bpins.test_key_gradients_sum_to_zero_and_value_gradients_to_the_output_gradients,
    bpins.test_window_zero_passes_the_gradient_to_v_only,
]


# Planted mistakes in the Transient-Global attention, caught by its pins.
from tests import test_oracle_tglobal as tpins  # noqa: E402

TG_MUTANTS = {
    "tg_side_bias_sign": ("longattn_oracle_t5_bucket(g - bi, num_buckets, max_distance)",
                          "longattn_oracle_t5_bucket(bi - g, num_buckets, max_distance)"),
    "tg_rms_without_sqrt": ("const double inv = 1.0 / sqrt(ms + eps);",
                            "const double inv = 1.0 / (ms + eps);"),
    "tg_window_short_on_the_right": ("const int64_t j1 = i + radius > n - 1 ? n - 1 : i + radius;",
                                     "const int64_t j1 = i + radius > n - 1 ? n - 1 : i + radius - 1;"),
    "tg_side_padding_ignored": ("if (key_pad && key_pad[b * n + i]) continue;", ""),
    "tg_log_ratio_swapped": ("const double x = log((double)a / (double)exact) / log((double)max_distance / (double)exact) *",
                             "const double x = log((double)max_distance / (double)exact) / log((double)a / (double)exact) *"),
    "tg_positive_half_swapped": ("const int64_t base = rel > 0 ? half : 0;",
                                 "const int64_t base = rel < 0 ? half : 0;"),
}

TG_PINS = [
    lambda: [tpins.test_bucket_matches_integer_statement(nb, md)
             for nb, md in [(32, 128), (16, 64)]],
    tpins.test_bucket_shape_of_the_rule,
    lambda: [tpins.test_side_tokens_match_brute_force(n, b)
             for n, b in [(70, 8), (64, 16), (5, 16), (33, 16)]],
    tpins.test_rms_norm_gives_unit_rms_and_the_tail_block_merges,
    lambda: [tpins.test_forward_matches_dense_brute_force(kw)
             for kw in [dict(), dict(radius=0), dict(pad_tail=(5, 40))]],
    tpins.test_without_bias_and_with_a_full_window_it_is_attention_over_concatenated_keys,
    lambda: tpins.test_entry_count_closed_form(300, 5, 8),
]


def _caught(lib_path, pins_list=None):
    failures = 0
    with oracle.substituted_library(lib_path):
        for pin in (PINS if pins_list is None else pins_list):
            try:
                pin()
            except (AssertionError, ValueError):
                failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutant_c), "-lm"], check=True, capture_output=True)
    assert _caught(str(so)) >= 1, f"no pin catches the planted mistake {name}"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_planted_backward_mistake_is_caught(name, tmp_path):
    old, new = BWD_MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutant_c), "-lm"], check=True, capture_output=True)
    assert _caught(str(so), BWD_PINS) >= 1, f"no pin catches the planted mistake {name}"


@pytest.mark.parametrize("name", sorted(TG_MUTANTS))
def test_planted_tglobal_mistake_is_caught(name, tmp_path):
    old, new = TG_MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    mutant_c = tmp_path / "mutant.c"
    mutant_c.write_text(src.replace(old, new))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutant_c), "-lm"], check=True, capture_output=True)
    assert _caught(str(so), TG_PINS) >= 1, f"no pin catches the planted mistake {name}"


def test_unmutated_copy_passes_every_pin(tmp_path):
    so = tmp_path / "libcopy.so"
    subprocess.run(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    SRC, "-lm"], check=True, capture_output=True)
    assert _caught(str(so)) == 0
    assert _caught(str(so), BWD_PINS) == 0
    assert _caught(str(so), TG_PINS) == 0
