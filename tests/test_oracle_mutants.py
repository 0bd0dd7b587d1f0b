"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/fs_oracle.c (on the CPU only),
builds it, and runs the pin suite (tests/test_oracle_pins.py) against it in a
subprocess.  The pins pass on the real oracle (that file's own run); here every
mutant must make at least one of them fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fs_oracle.c")

# (name, text in fs_oracle.c, replacement, which occurrence)
MUTANTS = [
    ("rope_turns_backwards", "out[2 * k] = x0 * c - x1 * s;", "out[2 * k] = x0 * c + x1 * s;", 0),
    ("rope_wrong_frequency", "-2.0 * (double)k / (double)d", "-1.0 * (double)k / (double)d", 0),
    ("window_edge_exclusive", "long long lo = i - p->window;", "long long lo = i - p->window + 1;", 0),
    ("candidates_overlap_window", "long long n = (i - p->window) / p->cell;",
     "long long n = (i - p->window + p->cell - 1) / p->cell;", 0),
    ("summary_wrong_divisor", "mean[e] /= (double)s;", "mean[e] /= (double)(s - 1);", 0),
    ("amax_last_not_max", "if (norm > best) best = norm;", "best = norm;", 0),
    ("ties_to_smaller_index", "if (x->cell > y->cell) return -1;", "if (x->cell < y->cell) return -1;", 0),
    ("recent_cells_dropped", "for (int c = n - p->n_recent; c < n; ++c)", "for (int c = n; c < n; ++c)", 0),
    ("score_unscaled", "order[t].key = dot / sqrt((double)d) +", "order[t].key = dot +", 0),
    ("prior_center_at_cell_start", "const double p_c = ((double)c + 0.5) * (double)p->cell;",
     "const double p_c = (double)c * (double)p->cell;", 0),
    ("prior_erf_scale_missing_2", "erf(((double)i - p_c) / (2.0 * sig))",
     "erf(((double)i - p_c) / sig)", 0),
    ("prior_offset_sign", "erf(((double)i - p_c) / (2.0 * sig))",
     "erf((p_c - (double)i) / (2.0 * sig))", 0),
    ("prior_drops_norm", "return lam * a_c * erf(", "return lam * erf(", 0),
    ("rerank_drops_log", "return mx + log(sum);", "return mx + sum;", 0),
    ("rerank_max_not_lse", "return mx + log(sum);", "return mx;", 0),
    ("rerank_unscaled_logits", "lg[t] = dot / sqrt((double)d);", "lg[t] = dot;", 0),
    ("readout_logits_unscaled", "logits[t] = dot / sqrt((double)d);", "logits[t] = dot;", 1),
    ("window_logits_unscaled", "logits[t] = dot / sqrt((double)d);", "logits[t] = dot;", 0),
    ("rmsnorm_drops_eps", "sqrt(ms + p->rms_eps)", "sqrt(ms)", 0),
    ("rmsnorm_sum_not_mean", "ms /= (double)d;", "ms /= 1.0;", 0),
    ("combine_drops_alpha", "o[e] = o_sr[e] + alpha * o_lr[e];", "o[e] = o_sr[e] + o_lr[e];", 0),
    ("softmax_unshifted_denominator", "den += exp(logits[t] - mx);", "den += exp(logits[t] - 0.5 * mx);", 0),
    ("topk_one_short", "int cnt = n_cand < p->topk ? n_cand : p->topk;",
     "int cnt = n_cand < p->topk ? n_cand : p->topk - 1;", 0),
    ("prune_one_short", "for (int r = 0; r < n && r < p->budget; ++r)",
     "for (int r = 0; r < n && r < p->budget - 1; ++r)", 0),
]


def _mutate(src: str, old: str, new: str, occ: int) -> str:
    pos = -1
    for _ in range(occ + 1):
        pos = src.find(old, pos + 1)
        assert pos >= 0, f"mutation site not found: {old!r} #{occ}"
    return src[:pos] + new + src[pos + len(old):]


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_kill_mutant(tmp_path, name, old, new, occ):
    src = open(SRC).read()
    mutated = _mutate(src, old, new, occ)
    assert mutated != src
    c_path = tmp_path / "fs_oracle.c"
    c_path.write_text(mutated)
    (tmp_path / "fs_oracle.h").write_text(open(os.path.join(ROOT, "oracle", "fs_oracle.h")).read())
    lib = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared", "-o", str(lib),
                           str(c_path), os.path.join(ROOT, "oracle", "fsb_oracle.c"),
                           os.path.join(ROOT, "oracle", "fsb_plain.c"), "-I",
                           str(tmp_path), "-lm", "-lpthread"])
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
