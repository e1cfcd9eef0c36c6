"""The pins catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of the oracle's C source (a wrong
index, a dropped term, a wrong sign or an operand mix-up), builds that copy in a
temporary directory and runs every pin on it: at least one pin must fail. The
real oracle is never modified. The mistakes cover the forward, the merge and
the backward.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle_attn.c")

MUTANTS = {
    "causal_off_by_one": ("if (causal && j > q_offset + i)", "if (causal && j >= q_offset + i)"),
    "q_offset_ignored": ("if (causal && j > q_offset + i)", "if (causal && j > i)"),
    "head_map_interleaved": ("{ return h / (Hq / Hkv); }", "{ return h % Hkv; }"),
    "scale_one_over_d": ("{ return 1.0 / sqrt((double)D); }", "{ return 1.0 / (double)D; }"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "lse_max_dropped": ("*lse_out = M + log(l);", "*lse_out = log(l);"),
    "no_normalisation": ("for (int64_t d = 0; d < D; ++d) o_row[d] /= l;", ""),
    "k_v_swapped_in_scores": ("(double)qi[d] * (double)kb[j * D + d]", "(double)qi[d] * (double)vb[j * D + d]"),
    "segment_batch_index": ("seg_k[b * Lk + j]", "seg_k[j]"),
    "segment_test_inverted": ("seg_q[b * Lq + i] != seg_k[b * Lk + j]", "seg_q[b * Lq + i] == seg_k[b * Lk + j]"),
    "merge_weight_mixup": ("(w1 * o1[r * D + d] + w2 * o2[r * D + d])", "(w1 * o1[r * D + d] + w1 * o2[r * D + d])"),
    "merge_sign": ("const double w1 = exp(l1 - M), w2 = exp(l2 - M);", "const double w1 = exp(M - l1), w2 = exp(l2 - M);"),
    "empty_row_nan": ("  if (nvis == 0) {\n    *lse_out = -INFINITY;", "  if (nvis < 0) {\n    *lse_out = -INFINITY;"),
    # backward
    "bwd_dq_jacobian_term_dropped": ("const double ds = w[j] * (dp - rsum);", "const double ds = w[j] * dp;"),
    "bwd_dq_v_for_k": ("out[d] += scale * ds * (double)kb[j * D + d];", "out[d] += scale * ds * (double)vb[j * D + d];"),
    "bwd_row_sum_unweighted": ("r += w[j] * dp;", "r += dp;"),
    "bwd_dk_jacobian_term_dropped": ("const double ds = p * (dp - rsum[row]);", "const double ds = p * dp;"),
    "bwd_dk_scale_dropped": ("dkj[d] += scale * ds * (double)qi[d];", "dkj[d] += ds * (double)qi[d];"),
    "bwd_dv_uses_ds": ("dvj[d] += p * (double)di[d];", "dvj[d] += ds * (double)di[d];"),
    "bwd_dkdv_own_head_only": ("for (int64_t h = g * n_rep; h < (g + 1) * n_rep; ++h) {",
                               "for (int64_t h = g * n_rep; h < g * n_rep + 1; ++h) {"),
    "bwd_dkdv_lse_unshifted": ("const double p = exp(scale * sd - lse[row]);", "const double p = exp(scale * sd);"),
    "bwd_dkdv_stats_rows_missed": ("need[t] = 1; break;", "need[t] = (r > 0); break;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, "mutation site not found: %s" % name
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(before, after))
    lib_path = str(tmp_path / "libmutant.so")
    oracle.compile_source(str(mutant_src), lib_path, werror=False)
    orc = oracle.Oracle(oracle.open_library(lib_path))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin.__name__)
    assert caught, "no pin caught mutant %s" % name
