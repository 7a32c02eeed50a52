"""Meta-test of the oracle pins: plant one plausible mistake at a time into a
copy of the oracle source (CPU only), build it, and check that the pin suite
fails against it.  A mutant that survives means a pin is missing."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "infllm_oracle.c")

# (name, exact source text, replacement)
MUTANTS = [
    ("window_one_short", "int64_t last = mini64(p + (int64_t)W, n_ctx - 1);",
     "int64_t last = mini64(p + (int64_t)W - 1, n_ctx - 1);"),
    ("window_includes_key", "for (int64_t i = p + 1; i <= last; ++i) {",
     "for (int64_t i = p; i <= last; ++i) {"),
    ("rep_score_one_head", "  for (int32_t g = 0; g < G; ++g) {\n    const int64_t qoff",
     "  for (int32_t g = 0; g < 1; ++g) {\n    const int64_t qoff"),
    ("unit_keys_keep_sinks", "*lo = maxi64(j * B, n_init);", "*lo = j * B;"),
    ("units_start_at_block0", "int64_t first_block = n_init / B;", "int64_t first_block = 0;"),
    ("eligible_strict", "if (lo <= t_last - W) e = u + 1;", "if (lo < t_last - W) e = u + 1;"),
    ("ties_higher_position", "return (x->pos > y->pos) - (x->pos < y->pos);",
     "return (x->pos < y->pos) - (x->pos > y->pos);"),
    ("ascending_scores", "if (x->score > y->score) return -1;\n  if (x->score < y->score) return 1;",
     "if (x->score < y->score) return -1;\n  if (x->score > y->score) return 1;"),
    ("repr_mean_not_sum", "repr[i * d + c] = acc;\n", "repr[i * d + c] = acc / (double)n_keep;\n"),
    ("mean_over_block", "repr[i * d + c] = acc / (double)(hi - lo);",
     "repr[i * d + c] = acc / (double)B;"),
    ("score_one_head", "  for (int32_t g = 0; g < G; ++g)\n    for (int64_t i = 0; i < L; ++i)",
     "  for (int32_t g = 0; g < 1; ++g)\n    for (int64_t i = 0; i < L; ++i)"),
    ("score_drops_last_query", "for (int64_t i = 0; i < L; ++i)\n      for (int32_t c = 0; c < d; ++c)\n        qsum[c]",
     "for (int64_t i = 0; i < L - 1; ++i)\n      for (int32_t c = 0; c < d; ++c)\n        qsum[c]"),
    ("window_excludes_query", "if (p > t - W) return 1;", "if (p > t - W && p < t) return 1;"),
    ("window_one_wider", "if (p > t - W) return 1;", "if (p >= t - W) return 1;"),
    ("unit_index_without_sink_offset", "int64_t u = p / B - n_init / B;", "int64_t u = p / B;"),
    ("no_causal", "if (p > t) return 0;\n  if (p < n_init)", "if (p > t + 1) return 0;\n  if (p < n_init)"),
    ("sink_off_by_one", "if (p < n_init) return 1;", "if (p <= n_init) return 1;"),
    ("unscaled_logits", "const double scale = 1.0 / sqrt((double)d);", "const double scale = 1.0;"),
    ("topk_keeps_one_less", "int64_t n_keep = mini64(k_m, e);\n  int64_t kept",
     "int64_t n_keep = mini64(k_m - 1, e);\n  int64_t kept"),
    ("lse_without_max", "lse[(int64_t)g * L + i] = m + log(denom);", "lse[(int64_t)g * L + i] = log(denom);"),
    ("rope_frequency_halved", "pow(theta, -2.0 * (double)c / (double)d)",
     "pow(theta, -1.0 * (double)c / (double)d)"),
    ("rope_sin_sign", "x[c] = x0 * cs - x1 * sn;", "x[c] = x0 * cs + x1 * sn;"),
    ("rope_interleaved_pairs", "const double x0 = x[c], x1 = x[c + h];\n    x[c] = x0 * cs - x1 * sn;\n    x[c + h] = x1 * cs + x0 * sn;",
     "const double x0 = x[2 * c % d], x1 = x[(2 * c + 1) % d];\n    x[2 * c % d] = x0 * cs - x1 * sn;\n    x[(2 * c + 1) % d] = x1 * cs + x0 * sn;"),
    ("context_lo_one_early", "const int64_t lo = maxi64(n_init, t0 - W + 1);",
     "const int64_t lo = maxi64(n_init, t0 - W);"),
    ("unit_position_ignores_slot", "return n_init + (int64_t)m * B + (p - (p / B) * B);",
     "return n_init + (p - (p / B) * B);"),
    ("local_after_units_missing", "if (p >= lo) return n_init + (int64_t)k_m * B + (p - lo);",
     "if (p >= lo) return n_init + (p - lo);"),
    ("query_kept_absolute", "rope_rotate(qv, d, rope_theta, (double)orc_context_pos(t, t0, sel, k_m, B, n_init, W));",
     "rope_rotate(qv, d, rope_theta, (double)t);"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: " + name
    mutant = tmp_path / "mutant.c"
    mutant.write_text(src.replace(old, new, 1))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", str(mutant),
                    "-o", str(so), "-lm"], check=True, capture_output=True)
    env = dict(os.environ, INFLLM_ORACLE_SO=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_workloads.py"),
                        os.path.join(ROOT, "tests", "test_oracle_rope.py"),
                        "-k", "not reduced"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, "mutant %s survived the pins:\n%s" % (name, r.stdout[-2000:])
