"""The pins catch plausible mistakes in the oracle (CPU only).

Each case copies sv_oracle.c, plants one mistake by text substitution (a
dropped term, a wrong sign, index or operand, a wrong tie rule), compiles the
copy into a temporary library and requires at least one pin to fail on it.
The oracle source itself is never modified.
"""

import os

import pytest

import oracle
import pins

MUTANTS = {
    "ratio_transposed": ("r = (qx == 0.0) ? INFINITY : px / qx;", "r = (px == 0.0) ? INFINITY : qx / px;"),
    "residual_sign": ("double d = pv - orc_prob(q, v);", "double d = orc_prob(q, v) - pv;"),
    "residual_no_clamp": ("return d > 0.0 ? d : 0.0;", "return d;"),
    "residual_drops_q": ("    if (!q) return pv;\n", "    q = NULL;\n    if (!q) return pv;\n"),
    "temperature_times": ("exp((orc_load(base, dtype, off + (size_t)v) - m) / T)",
                          "exp((orc_load(base, dtype, off + (size_t)v) - m) * T)"),
    "prob_unnormalised": ("- r->m) / r->T) / r->s;", "- r->m) / r->T);"),
    "lse_drops_temperature": ("return r->m / r->T + log(r->s);", "return r->m + log(r->s);"),
    "accept_wrong_draw": ("double u = (double)u_accept[(size_t)b * K + i];",
                          "double u = (double)u_sample[(size_t)b * (K + 1) + i];"),
    "reject_does_not_stop": ("            if (!(u < r)) {\n                n = i;\n                break;\n            }",
                             "            if (!(u < r)) {\n                n = i;\n            }"),
    "sample_wrong_row": ("orc_row_init(&p, target, tbase + (size_t)n * V, dtype, V, T);\n        double us",
                         "orc_row_init(&p, target, tbase + (size_t)0 * V, dtype, V, T);\n        double us"),
    "sample_unnormalised": ("double t = u * Z;", "double t = u;"),
    "bonus_from_draft_row": ("orc_row_init(&q, draft, dbase + (size_t)n * V, dtype, V, T);",
                             "orc_row_init(&q, draft, dbase + (size_t)(n > 0 ? n - 1 : 0) * V, dtype, V, T);"),
    "argmax_last_on_ties": ("        if (x > bv) {", "        if (x >= bv) {"),
    "greedy_wrong_compare": ("if (i == K || x[i] != a) {", "if (i == K || x[i] == a) {"),
    "greedy_emits_draft": ("    tok[n] = a;\n", "    tok[n] = n < K ? x[n] : a;\n"),
    "tree_ignores_parent_ok": ("ok[j] = ok[p] && tk[j] == am[p];", "ok[j] = tk[j] == am[p];"),
    "tree_own_row": ("ok[j] = ok[p] && tk[j] == am[p];", "ok[j] = ok[p] && tk[j] == am[j];"),
    "tree_highest_on_ties": ("if (ok[j] && depth[j] > depth[best]) best = j;",
                             "if (ok[j] && depth[j] >= depth[best]) best = j;"),
    "tree_bonus_parent_row": ("out[d] = am[best];", "out[d] = am[par[best] < 0 ? 0 : par[best]];"),
    # the draw margins, which decide the flagged requests
    "margin_drops_left_edge": ("*margin = a < b ? a : b;", "*margin = b;"),
    "margin_drops_right_edge": ("*margin = a < b ? a : b;", "*margin = a;"),
    "margin_unnormalised": ("double a = fabs(u - Cprev / Z), b = fabs(u - C / Z);",
                            "double a = fabs(t - Cprev), b = fabs(t - C);"),
    "margin_skips_accept_draws": ("double d = fabs(u - r);", "double d = INFINITY;"),
    "margin_clamped_ratio": ("double d = fabs(u - r);", "double d = fabs(u - (r < 1.0 ? r : 1.0));"),
    "margin_skips_rejecting_draw": ("            if (isfinite(r)) {", "            if (isfinite(r) && u < r) {"),
    "margin_skips_sample_draw": ("        if (m2 < mg) mg = m2;\n", ""),
    "margin_fallback_not_boundary": ("                t = orc_inverse_cdf(&p, NULL, us, &m2, &Z);\n                m2 = 0.0;",
                                     "                t = orc_inverse_cdf(&p, NULL, us, &m2, &Z);"),
}


def _run_battery(lib):
    failures = []
    for pin in pins.ALL_FAST:
        try:
            pin(lib)
        except (AssertionError, RuntimeError, ValueError, IndexError) as e:
            failures.append(pin.__name__)
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(oracle.SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    so = str(tmp_path / f"libmut_{name}.so")
    oracle.build(str(path), so)
    lib = oracle.load(so)
    failures = _run_battery(lib)
    assert failures, f"no pin detected mutant {name}"


def test_unmutated_passes_battery(olib):
    assert _run_battery(olib) == []
