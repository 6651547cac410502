"""Planted mistakes: each one is a plausible slip in the oracle (a dropped term,
a wrong sign or index, a swapped operand).  It is applied to a temporary copy
of oracle.c, compiled on the CPU, and the pins must reject every such build.
The real oracle.c is never modified."""
import os
import subprocess
import sys

import pytest

import oracle as O
from tests import test_oracle_pins as P

SRC = os.path.join(os.path.dirname(O.__file__), "oracle.c")

MUTANTS = {
    "rope_sign": ("v[2 * i] = a * c[i] - b * s[i];", "v[2 * i] = a * c[i] + b * s[i];"),
    "rope_frequency_width": ("pow(base, -2.0 * (double)i / (double)dh)", "pow(base, -2.0 * (double)i / (double)(2 * dh))"),
    "rope_missing_on_q": ("o_rope_apply(q, R, H, dh, pos_q, cos_tab, sin_tab);", ""),
    "k_position_off_by_one": ("pos_k[(int64_t)b * T + t] = s0 + t;", "pos_k[(int64_t)b * T + t] = s0 + t + 1;"),
    "causal_diagonal_excluded": ("p + 1, dh, scale", "p, dh, scale"),
    "gqa_tiled_not_interleaved": ("int kvh = hd / group;", "int kvh = hd % Hkv;"),
    "score_scale_dropped": ("s[j] = dot * scale;", "s[j] = dot;"),
    "softmax_not_normalised": ("float p = s[j] / z;", "float p = s[j];"),
    "keys_reversed": ("const float *kj = kc + (int64_t)j * dh;", "const float *kj = kc + (int64_t)(n_keys - 1 - j) * dh;"),
    "residual_dropped": ("r[i] = xs[i] + a[i];", "r[i] = a[i];"),
    "second_residual_dropped": ("out[i] = r[i] + m[i];", "out[i] = m[i];"),
    "gate_up_swapped": ("gate[i] = silu(gate[i]) * up[i];", "gate[i] = silu(up[i]) * gate[i];"),
    "rms_gain_dropped": ("y[i] = x[i] * r * g[i];", "y[i] = x[i] * r;"),
    "rms_eps_outside_sqrt": ("float r = 1.0f / sqrtf(ms + eps);", "float r = 1.0f / (sqrtf(ms) + eps);"),
    "rms_mean_over_wrong_width": ("float ms = ss / (float)d;", "float ms = ss / (float)(d - 1);"),
    "wrong_weight_in_out_proj": ("o_matmul(att, w->wo, R, qd, d, a, cnt);", "o_matmul(att, w->wq, R, qd, d, a, cnt);"),
    "cache_layout_b_g_swapped": ("int64_t dst = (((int64_t)b * Hkv + g) * t_max + p) * dh;",
                                 "int64_t dst = (((int64_t)g * B + b) * t_max + p) * dh;"),
    "matmul_transposed_operand": ("const float *wr = w + (int64_t)p * n;", "const float *wr = w + (int64_t)(k - 1 - p) * n;"),
    # bf16 storage: a rounding of a GEMM operand dropped, misplaced or wrong
    "bf16_att_not_rounded": ("    operand_round(cfg, att, R * qd);\n", ""),
    "bf16_k_not_rounded": ("    operand_round(cfg, k, M * kvd);\n", ""),
    "bf16_act_not_rounded": ("    operand_round(cfg, gate, R * f);", ""),
    "bf16_q_rounded_before_rope": (
        "    o_rope_apply(q, R, H, dh, pos_q, cos_tab, sin_tab);\n    o_rope_apply(k, M, Hkv, dh, pos_k, cos_tab, sin_tab);\n",
        "    operand_round(cfg, q, R * qd);\n    o_rope_apply(q, R, H, dh, pos_q, cos_tab, sin_tab);\n"
        "    o_rope_apply(k, M, Hkv, dh, pos_k, cos_tab, sin_tab);\n"),
    # the value handed out as "before rounding" is taken after it
    "bf16_pre_value_after_rounding": (
        "    if (inter && inter->act_pre) memcpy(inter->act_pre, gate, sizeof(float) * R * f);\n"
        "    operand_round(cfg, gate, R * f);",
        "    operand_round(cfg, gate, R * f);\n"
        "    if (inter && inter->act_pre) memcpy(inter->act_pre, gate, sizeof(float) * R * f);"),
    # cache append
    "kv_append_row_off_by_one": ("int64_t dst = (((int64_t)b * Hkv + g) * t_max + start[b] + t) * dh;",
                                 "int64_t dst = (((int64_t)b * Hkv + g) * t_max + start[b] + t + 1) * dh;"),
    "kv_append_source_heads_swapped": ("int64_t src = (((int64_t)b * n_new + t) * Hkv + g) * dh;",
                                       "int64_t src = (((int64_t)b * Hkv + g) * n_new + t) * dh;"),
    "bf16_round_truncates": ("u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0u;"),
    "bf16_layer_output_not_rounded": ("operand_round(cfg, y, (last ? (int64_t)B * n_rows : M) * d);", ""),
    "bf16_final_norm_not_rounded": ("operand_round(cfg, hn, R * d);", ""),
    # sliding window
    "window_off_by_one": ("int j0 = p - window + 1;", "int j0 = p - window;"),
    "window_ignored_in_block": ("const int j0 = o_window_first_key(p, cfg->window);", "const int j0 = 0;"),
}

PINS = [
    P.test_block_matches_fp64_library_composition,
    P.test_bf16_operands_match_fp64_composition,
    P.test_bf16_model_matches_fp64_composition,
    P.test_sliding_window_first_key_matches_page_example,
    P.test_sliding_window_attention_reads_exactly_the_window,
    P.test_sliding_window_block_matches_fp64_band_mask,
    P.test_decode_matches_fp64_library_composition,
    P.test_decode_equals_prefill_bitwise,
    P.test_gqa_equals_mha_with_repeated_kv_bitwise,
    P.test_rms_norm_closed_form,
    P.test_rope_properties,
    P.test_attention_closed_forms,
    P.test_softmax_rows_sum_to_one,
    P.test_values_before_rounding,
    P.test_kv_append_places_every_value,
    P.test_kv_append_equals_the_block_cache_write,
]


def _caught(orc) -> list:
    hits = []
    for pin in PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            hits.append(pin.__name__)
    return hits


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, "mutation anchor must match exactly once"
    src = tmp_path / "oracle_mut.c"
    src.write_text(text.replace(old, new))
    so = O.build(src=str(src), out=str(tmp_path / "liboracle_mut.so"))
    # A planted mistake may also corrupt memory, so the pins run in a child
    # process; a crash there counts as caught.
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import oracle as O\n"
            "from tests.test_oracle_mutants import _caught\n"
            "print('HITS', len(_caught(O.Oracle(%r))))\n") % (root, so)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True)
    caught = res.returncode != 0 or "HITS 0" not in res.stdout
    assert caught, "planted mistake %r passed every pin" % name


def test_unmutated_build_passes_every_pin(tmp_path):
    so = O.build(out=str(tmp_path / "liboracle_copy.so"))
    assert _caught(O.Oracle(so)) == []
