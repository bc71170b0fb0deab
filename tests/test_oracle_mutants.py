"""Plant mistakes in copies of the oracle (CPU only) and check the pins catch each.

Every mutant is the oracle source with one plausible slip -- a dropped term, a
wrong sign or index, a swapped operand, a reversed tie rule, an off-by-one in
the window -- compiled to a temporary library.  At least one pin in
oracle_pins.ALL_PINS must fail on it; otherwise the pins would not notice that
mistake in the real oracle either.
"""
import os
import shutil
import subprocess

import pytest

import oracle as O
import oracle_pins as P
from oracle.build import CFLAGS, HERE

SRC = os.path.join(HERE, "h2o_oracle.c")

MUTANTS = {
    "drop_scale": ("s *= u->c.scale;", ""),
    "softmax_sign": ("exp(u->w[i] - m)", "exp(m - u->w[i])"),
    "value_rows_are_keys": ("const double *vj = u->V +", "const double *vj = u->K +"),
    "slot_index_for_position": ("const double *kj = u->K + (size_t)u->R[i] * D;",
                                "const double *kj = u->K + (size_t)i * D;"),
    "score_only_first_query_head": ("        if (scored)\n            for (int i = 0; i < n; ++i) u->score[u->R[i]] += u->w[i];",
                                    "        if (scored && g == 0)\n            for (int i = 0; i < n; ++i) u->score[u->R[i]] += u->w[i];"),
    "score_missing_new_token": ("for (int i = 0; i < n; ++i) u->score[u->R[i]] += u->w[i];",
                                "for (int i = 0; i < n - 1; ++i) u->score[u->R[i]] += u->w[i];"),
    "tie_keeps_higher_position": ("    return (x->pos > y->pos) ? -1 : (x->pos < y->pos) ? 1 : 0;\n}\n\nstatic int cmp_key",
                                  "    return (x->pos < y->pos) ? -1 : (x->pos > y->pos) ? 1 : 0;\n}\n\nstatic int cmp_key"),
    "evict_highest_score": ("    if (x->score < y->score) return -1;\n    if (x->score > y->score) return 1;",
                            "    if (x->score > y->score) return -1;\n    if (x->score < y->score) return 1;"),
    "recent_window_off_by_one": ("if (p >= u->c.n_sink && p < len - W) {", "if (p >= u->c.n_sink && p <= len - W) {"),
    "sink_off_by_one": ("if (p >= u->c.n_sink && p < len - W) {", "if (p > u->c.n_sink && p < len - W) {"),
    "evict_count_off_by_one": ("        e = n - K;\n", "        e = n - K - 1;\n"),
    "hh_split_rounds_up": ("hh = (k - c->n_sink) / 2;", "hh = (k - c->n_sink + 1) / 2;"),
    "philox_key_word": ("uint64_t y0 = hi1 ^ x1 ^ k0", "uint64_t y0 = hi1 ^ x1 ^ k1"),
    "philox_weyl_before_first_round": ("        if (r > 0) {\n            k0 += W0;", "        if (r >= 0) {\n            k0 += W0;"),
    "random_evicts_prompt": ("if (u->R[i] >= u->prompt_len) {", "if (u->R[i] >= 0) {"),
    "random_counter_step_word": ("(uint64_t)u->h, (uint64_t)t,", "(uint64_t)u->h, (uint64_t)(t + 1),"),
    "colsum_rows_from_zero": ("for (int i = row_lo; i < P && rc == ORC_OK; ++i)",
                              "for (int i = 0; i < P && rc == ORC_OK; ++i)"),
    "colsum_no_scale": ("w[j] = scale * s;", "w[j] = s;"),
    "colsum_first_head_only": ("for (int g = 0; g < G; ++g) {\n            const double *qi",
                               "for (int g = 0; g < 1; ++g) {\n            const double *qi"),
    "colsum_key_is_query_row": ("const double *kj = k + (size_t)j * D;", "const double *kj = k + (size_t)i * D;"),
    "colsum_head_major_query": ("const double *qi = q + ((size_t)i * G + g) * D;",
                                "const double *qi = q + ((size_t)g * P + i) * D;"),
    "snapkv_pool_radius": ("const int Pp = P - w, r = pool / 2;", "const int Pp = P - w, r = pool / 2 + 1;"),
    "snapkv_ties_keep_higher": ("    return (x->pos < y->pos) ? -1 : (x->pos > y->pos) ? 1 : 0;\n}\n\nint orc_snapkv_select",
                                "    return (x->pos > y->pos) ? -1 : (x->pos < y->pos) ? 1 : 0;\n}\n\nint orc_snapkv_select"),
    "snapkv_drop_window": ("    for (int j = Pp; j < P; ++j) mark[j] = 1;\n", ""),
    "snapkv_pool_into_window": ("if (x >= 0 && x < Pp && vg[x] > m)", "if (x >= 0 && x < P && vg[x] > m)"),
    "snapkv_lowest_votes": ("    if (x->v > y->v) return -1;\n    if (x->v < y->v) return 1;",
                            "    if (x->v < y->v) return -1;\n    if (x->v > y->v) return 1;"),
    "snapkv_first_head_only": ("for (int g = 0; g < G; ++g) {\n        const double *vg",
                               "for (int g = 0; g < 1; ++g) {\n        const double *vg"),
    "block_evict_most_important": ("    if (x->imp != y->imp) return x->imp < y->imp ? -1 : 1;",
                                   "    if (x->imp != y->imp) return x->imp > y->imp ? -1 : 1;"),
    "block_ties_newer_first": ("    return (x->block < y->block) ? -1 : (x->block > y->block) ? 1 : 0;",
                               "    return (x->block > y->block) ? -1 : (x->block < y->block) ? 1 : 0;"),
    "block_sink_block_eligible": ("cand[k] = full && lo >= c->n_sink && hi < len - W;",
                                  "cand[k] = full && hi >= c->n_sink && hi < len - W;"),
    "block_window_off_by_one": ("cand[k] = full && lo >= c->n_sink && hi < len - W;",
                                "cand[k] = full && lo >= c->n_sink && hi <= len - W;"),
    "block_holes_ignored": ("full = live[p] != 0;", "full = 1;"),
    "block_first_head_only": ("    for (int i = 0; i < n_units; ++i) {\n        const double *sc = scores",
                              "    for (int i = 0; i < 1; ++i) {\n        const double *sc = scores"),
    "block_hh_plus_one": ("const int hh = HH < nt ? HH : nt;\n        for (int x = 0; x < hh; ++x) imp",
                          "const int hh = HH + 1 < nt ? HH + 1 : nt;\n        for (int x = 0; x < hh; ++x) imp"),
    "block_counts_lowest_scores": ("imp[tok[x].pos / page] += 1;", "imp[tok[nt - 1 - x].pos / page] += 1;"),
    "block_need_rounds_down": ("const int need = (n - K + page - 1) / page;", "const int need = (n - K) / page;"),
    "block_select_own_scores_first_unit": ("memcpy(sc + (size_t)i * len, u[i]->score,", "memcpy(sc + (size_t)i * len, u[0]->score,"),
    "step_many_skips_units": ("for (int i = j->first; i < j->n; i += j->stride)",
                              "for (int i = j->first; i < j->n; i += 2 * j->stride)"),
    "decay_not_applied": ("for (int i = 0; i < n; ++i) u->score[u->R[i]] *= lam;",
                          "for (int i = 0; i < n; ++i) u->score[u->R[i]] *= 1.0;"),
    "decay_per_query_head": ("            for (int i = 0; i < n; ++i) u->score[u->R[i]] += u->w[i];",
                             "            for (int i = 0; i < n; ++i) u->score[u->R[i]] = lam * u->score[u->R[i]] + u->w[i];"),
    "decay_squared": ("u->score[u->R[i]] *= lam;", "u->score[u->R[i]] *= lam * lam;"),
    "f16_rounds_toward_zero": ("return copysign(rint(a / q) * q, x);", "return copysign(floor(a / q) * q, x);"),
    "f16_ties_away_from_zero": ("return copysign(rint(a / q) * q, x);", "return copysign(round(a / q) * q, x);"),
    "f16_no_subnormal_floor": ("    if (e < -14) e = -14;\n", ""),
    "f16_overflow_saturates": ("if (a >= 65520.0) return copysign(INFINITY, x);", "if (a >= 65520.0) return copysign(65504.0, x);"),
    "f16_eleven_fraction_bits": ("const double q = ldexp(1.0, e - 10);", "const double q = ldexp(1.0, e - 11);"),
    "f16_scores_not_rounded": ("        for (int i = 0; i < n; ++i) u->score[u->R[i]] = orc_round_f16(u->score[u->R[i]]);",
                               "        for (int i = 0; i < n; ++i) u->score[u->R[i]] = u->score[u->R[i]];"),
    "f16_initial_scores_not_rounded": ("        if (u->c.score_f16) u->score[p] = orc_round_f16(u->score[p]);\n", ""),
    "random_largest_words": ("    if (x->key < y->key) return -1;\n    if (x->key > y->key) return 1;",
                             "    if (x->key > y->key) return -1;\n    if (x->key < y->key) return 1;"),
}


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    d = tmp_path_factory.mktemp("oracle_mutants")
    shutil.copy(os.path.join(HERE, "h2o_oracle.h"), d / "h2o_oracle.h")
    return d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique in the oracle"
    path = mutant_dir / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib_path = str(mutant_dir / f"lib{name}.so")
    subprocess.run(["gcc", *CFLAGS, "-I", str(mutant_dir), "-o", lib_path, str(path), "-lm"],
                   check=True, capture_output=True)
    lib = O.load(lib_path)
    for pin in P.ALL_PINS:
        try:
            pin(lib)
        except (AssertionError, O.OracleError):
            return
    pytest.fail(f"no pin caught mutant {name}")
