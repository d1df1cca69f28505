"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/hetattn_oracle.c`` (on the
CPU, in a temporary directory), builds it, and runs the oracle pin tests
against the copy.  The pins pass on the real oracle; here at least one must
fail for every planted mistake.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "hetattn_oracle.c")

MUTANTS = {
    "window_centre_off_by_one": ("int s = pos - (k - 1) / 2;", "int s = pos - (k + 1) / 2;"),
    "window_not_shifted_at_far_border": ("if (s > S - L) s = S - L;", ""),
    "ties_to_higher_index": ("return (a->idx < b->idx) ? -1 : (a->idx > b->idx) ? 1 : 0;",
                             "return (a->idx < b->idx) ? 1 : (a->idx > b->idx) ? -1 : 0;"),
    "rho_n_truncated": ("floor(rho * (double)N + 0.5)", "floor(rho * (double)N)"),
    "mean_std_non_strict": ("(mapped_u(ub[i]) < T) ? 0 : 1", "(mapped_u(ub[i]) <= T) ? 0 : 1"),
    "sample_std": ("sqrt(ss / (double)N)", "sqrt(ss / (double)(N - 1))"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "key_row_stride": ("const float *kr = kbase + (long)keys[j] * key_stride;",
                       "const float *kr = kbase + (long)keys[j] * D;"),
    "window_axes_swapped": ("oracle_window_axis(Hg, wh, y, &y0, &ly);",
                            "oracle_window_axis(Hg, ww, y, &y0, &ly);"),
    "nan_least_uncertain": ("if (isnan(x)) return INFINITY;", "if (isnan(x)) return -INFINITY;"),
    "value_from_query_row": ("const float *vr = vbase + (long)keys[j] * key_stride;",
                             "const float *vr = vbase;"),
    "local_mask_inverted": ("if (!is_local) {", "if (is_local) {"),
    # per-block random swap and its generator
    "philox_weyl_constant": ("W1 = 0xBB67AE85u", "W1 = 0xBB67AE86u"),
    "philox_key_not_bumped_first_round_too": ("if (round > 0) {", "if (round >= 0) {"),
    "swap_largest_keys": ("if (a->key < b->key) return -1;\n    if (a->key > b->key) return 1;",
                          "if (a->key < b->key) return 1;\n    if (a->key > b->key) return -1;"),
    "swap_ratio_truncated": ("floor(r * (double)N + 0.5)", "floor(r * (double)N)"),
    "swap_counter_words_swapped": ("{(unsigned int)i, (unsigned int)b, block, step}",
                                   "{(unsigned int)i, (unsigned int)b, step, block}"),
    "swap_not_capped_by_local_set": ("if (S > nl) S = nl;", ""),
    "swap_ties_higher_index_first": ("return (a->idx < b->idx) ? -1 : 1;",
                                     "return (a->idx < b->idx) ? 1 : -1;"),
    # ablation routers and the cut window border
    "uniform_lattice_ends_segments": ("dense[j * (long)N / K] = 1;",
                                      "dense[(j * (long)N + K - 1) / K] = 1;"),
    # backward pass
    "backward_drops_row_term": ("const double ds = s[j] * (w[j] - Dsum);", "const double ds = s[j] * w[j];"),
    "backward_dk_without_scale": ("dkr[d] += scale * ds * (double)qrow[d];", "dkr[d] += ds * (double)qrow[d];"),
    "backward_dv_uses_ds": ("dvr[d] += s[j] * (double)dorow[d];", "dvr[d] += ds * (double)dorow[d];"),
    "kv_rows_window_far_edge_included": ("if (pos_j[ax] < start || pos_j[ax] >= start + len) return 0;",
                                         "if (pos_j[ax] < start || pos_j[ax] > start + len) return 0;"),
    "kv_rows_drops_row_term": ("const double ds = p * (dp - dsum[n * nh + i]);", "const double ds = p * dp;"),
    "router_count_truncated": ("floor((double)N * rho + 0.5)", "floor((double)N * rho)"),
    "random_largest_draws": ("for (long j = 0; j < K; j++) dense[tok[j].idx] = 1;",
                             "for (long j = 0; j < K; j++) dense[tok[N - 1 - j].idx] = 1;"),
    "cut_window_short_high_side": ("int lo = pos - h, hi = pos + h + 1;", "int lo = pos - h, hi = pos + h;"),
    "cut_border_uses_shifted_window": ("    if (border == 0) {\n        oracle_window_axis(T,",
                                       "    if (border >= 0) {\n        oracle_window_axis(T,"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    mutant = tmp_path / "hetattn_oracle.c"
    mutant.write_text(src.replace(old, new))
    (tmp_path / "hetattn_oracle.h").write_text(open(SRC[:-1] + "h").read())
    lib = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w",
                           str(mutant), "-o", str(lib), "-lm"])
    env = dict(os.environ, HETATTN_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_route.py"),
                        os.path.join(ROOT, "tests", "test_oracle_attention.py"),
                        os.path.join(ROOT, "tests", "test_oracle_swap.py"),
                        os.path.join(ROOT, "tests", "test_oracle_variants.py"),
                        os.path.join(ROOT, "tests", "test_oracle_backward.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin:\n{r.stdout[-2000:]}"
