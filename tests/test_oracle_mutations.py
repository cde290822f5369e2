"""The oracle's pins catch planted mistakes.

Each case copies oracle/skinny_oracle.c, plants one plausible mistake (a
dropped term, a transposed operand, a wrong tie rule, bias, divisor, nibble
order, ...), compiles the copy with gcc and runs the pin battery of
tests/test_oracle_*.py against it.  At least one pin must fail for every
mistake; the unmodified copy must pass them all.  Everything here runs on
the CPU.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_formats as F
from tests import test_oracle_gemm as G
from tests import test_oracle_norm as Nm
from tests import test_oracle_publish as Pb
from tests import test_oracle_dual_norm as Dn

SRC = os.path.join(os.path.dirname(oracle.__file__), "skinny_oracle.c")

# (name, text in the source, replacement)
MUTATIONS = [
    ("gemm_drops_last_term",
     "      for (int k = 0; k < K; ++k)\n        acc += oracle_bf16_value(x[(size_t)m * K + k]) *",
     "      for (int k = 0; k < K - 1; ++k)\n        acc += oracle_bf16_value(x[(size_t)m * K + k]) *"),
    ("gemm_transposed_w", "oracle_bf16_value(w[(size_t)n * K + k]);\n      y[",
     "oracle_bf16_value(w[(size_t)k * N + n]);\n      y["),
    ("gemm_output_transposed", "y[(size_t)m * N + n] = oracle_bf16_round(acc);",
     "y[(size_t)n * M + m] = oracle_bf16_round(acc);"),
    ("bf16_ties_away", "double q = nearbyint(ldexp(a, 8 - e));", "double q = round(ldexp(a, 8 - e));"),
    ("bf16_truncates", "double q = nearbyint(ldexp(a, 8 - e));", "double q = floor(ldexp(a, 8 - e));"),
    ("ties_to_odd_code", "(c & 1) == 0 && (best & 1) == 1", "(c & 1) == 1 && (best & 1) == 0"),
    ("e4m3_wrong_bias", "mag = ldexp(1.0 + man / 8.0, exp - 7);", "mag = ldexp(1.0 + man / 8.0, exp - 8);"),
    ("e2m1_drops_sign", "return (uint8_t)(signbit(v) ? 0x8 | mag : mag);", "return (uint8_t)mag;"),
    ("block_scale_over_4", "global_scale * amax / 6.0", "global_scale * amax / 4.0"),
    ("output_scale_inverted", "global_scale / dec; /* [oscale] */", "dec / global_scale; /* [oscale] */"),
    ("signed_amax", "if (fabs(yn[j]) > amax) amax = fabs(yn[j]);", "if (yn[j] > amax) amax = yn[j];"),
    ("nibbles_swapped", "(uint8_t)(codes[2 * i] | (codes[2 * i + 1] << 4));",
     "(uint8_t)(codes[2 * i + 1] | (codes[2 * i] << 4));"),
    ("mean_over_p_minus_1", "double inv = 1.0 / sqrt(ss / P + eps);",
     "double inv = 1.0 / sqrt(ss / (P - 1) + eps);"),
    ("eps_outside_root", "double inv = 1.0 / sqrt(ss / P + eps);",
     "double inv = 1.0 / (sqrt(ss / P) + eps);"),
    ("gain_center_dropped", "(oracle_bf16_value(w[j]) + gain_center)", "oracle_bf16_value(w[j])"),
    ("publish_keeps_negative_zero", "(v == 0x8000u) ? 0x0000u : v;", "v;"),
    ("publish_zeroes_every_sign", "(v == 0x8000u) ? 0x0000u : v;", "v & 0x7FFFu;"),
    ("publish_rank_stage_swapped", "((size_t)stage * tp + rank)", "((size_t)rank * 3 + stage)"),
    ("publish_ticket_low_half", "(int)((uint32_t)ticket[0] >> 16)", "(int)((uint32_t)ticket[0] & 0xFFFF)"),
    ("publish_sets_next_stage", "if (!ticket) stage_state[1] = stage;", "if (!ticket) stage_state[0] = stage;"),
    ("publish_word_with_ticket", "if (!ticket) stage_state[1] = stage;", "if (stage_state) stage_state[1] = stage;"),
    ("dual_drops_beta_term", "a * (double)st[j] + oracle_bf16_value(beta[j]) * oracle_bf16_value(h);",
     "a * (double)st[j];"),
    ("dual_alpha_on_h", "a * (double)st[j] + oracle_bf16_value(beta[j]) * oracle_bf16_value(h);",
     "(double)st[j] + oracle_bf16_value(beta[j]) * a * oracle_bf16_value(h);"),
    ("dual_pre_uses_post_eps", "double inv2 = 1.0 / sqrt(ss2 / H + pre_eps);",
     "double inv2 = 1.0 / sqrt(ss2 / H + post_eps);"),
    ("dual_pre_drops_gain_center", "(oracle_bf16_value(next_w[j]) + pre_gc));",
     "oracle_bf16_value(next_w[j]));"),
    ("dual_gc_without_weight", "post_w ? oracle_bf16_value(post_w[j]) + post_gc : 1.0;",
     "post_w ? oracle_bf16_value(post_w[j]) + post_gc : 1.0 + post_gc;"),
    ("dual_h_not_rounded", "st[j] = (float)v;", "st[j] = (float)(a * (double)st[j] + oracle_bf16_value(beta[j]) * oracle_bf16_value(p[j]) * inv * g);"),
]

# The pins (test functions that raise AssertionError on a mismatch).
BATTERY = [
    lambda: [G.test_gemm_brute_force_rational(s) for s in range(4)],
    G.test_gemm_midpoint_ties,
    G.test_gemm_identity_and_one_hot,
    G.test_gemm_non_square_orientation,
    G.test_gemm_exact_sums_match_numpy_float64,
    G.test_gemm_exact_integer_inputs,
    F.test_bf16_roundtrip_every_pattern,
    F.test_bf16_round_matches_torch_from_float32,
    F.test_bf16_round_exact_rational_midpoints,
    F.test_e4m3_decode_matches_torch,
    F.test_e4m3_encode_matches_torch_in_range,
    F.test_e4m3_saturates_and_roundtrips,
    F.test_e2m1_decode_table,
    lambda: [F.test_e2m1_ties_and_saturation(v, c) for v, c in
             [(0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6),
              (5.0, 0x6), (1e9, 0x7), (-0.25, 0x8), (-5.0, 0xE)]],
    lambda: [Nm.test_golden_worked_blocks(c) for c in Nm._parse_golden()],
    Nm.test_rmsnorm_constant_row_closed_form,
    Nm.test_rmsnorm_one_hot_closed_form,
    Nm.test_global_max_block_hits_the_largest_codes,
    Nm.test_all_zero_block,
    Nm.test_packing_low_nibble_even_column,
    Pb.test_publish_worked_case,
    Pb.test_publish_ticket_stage_uses_upper_half_and_stores_no_word,
    lambda: [Pb.test_publish_outside_stages_writes_nothing(s, t) for s, t in
             [([3, 7], None), ([-1, 7], None), (None, [3 << 16]), (None, [0x7FFF0000])]],
    lambda: [Pb.test_publish_properties(k) for k in range(6)],
    Dn.test_identity_gate_keeps_stream_and_normalises_it,
    Dn.test_beta_gate_replaces_stream_with_post_norm,
    Dn.test_post_norm_without_weight_one_hot,
    lambda: [Dn.test_gated_add_exact_small_numbers(a) for a in (False, True)],
    Dn.test_pre_norm_reads_the_updated_stream,
    Dn.test_rows_are_independent,
]


def _build(tmp_path, name, text=None, repl=None):
    with open(SRC) as f:
        src = f.read()
    if text is not None:
        assert src.count(text) >= 1, f"mutation {name}: pattern not in the oracle source"
        src = src.replace(text, repl)
    c = tmp_path / f"{name}.c"
    c.write_text(src)
    so = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
                    str(c), "-o", str(so), "-lm"], check=True)
    return oracle.load_library(str(so))


def _failures(lib):
    failed = []
    with oracle.use_library(lib):
        for i, pin in enumerate(BATTERY):
            try:
                pin()
            except AssertionError:
                failed.append(i)
    return failed


def test_unmodified_copy_passes_every_pin(tmp_path):
    assert _failures(_build(tmp_path, "unmodified")) == []


@pytest.mark.parametrize("name,text,repl", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(tmp_path, name, text, repl):
    failed = _failures(_build(tmp_path, name, text, repl))
    assert failed, f"no pin catches the planted mistake '{name}'"
