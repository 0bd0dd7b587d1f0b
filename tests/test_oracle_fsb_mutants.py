"""The FS-B oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/fsb_oracle.c (the
fixed-order oracle) or oracle/fsb_plain.c (the plain fp64 one), on the CPU
only, builds it with the other unchanged sources, and runs
tests/test_oracle_fsb_pins.py against it in a subprocess; every mutant must
make at least one pin fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SOURCES = ("fs_oracle.c", "fsb_oracle.c", "fsb_plain.c")

# (name, text in fsb_oracle.c, replacement)
MUTANTS = [
    ("radius_term_dropped", "t = t * (double)f->rho[node];", "t = 0.0;"),
    ("radius_without_query_norm", "double t = slack * q_norm;", "double t = slack;"),
    ("mean_not_divided", "(float)(sum[e] * ldexp(1.0, -l))", "(float)(sum[e])"),
    ("radius_of_last_leaf", "if (acc > r2) r2 = acc;", "r2 = acc;"),
    ("node_norm_of_first_leaf", "if (amax[c] > a_best) a_best = amax[c];", "a_best = amax[c];"),
    ("children_not_doubled", "e.index = 2 * cur[t].index + ch;", "e.index = cur[t].index + ch;"),
    ("roots_unaligned", "index[cnt] = start >> l;", "index[cnt] = start;"),
    ("ties_to_earlier_block", "if (x->first > y->first) return -1;", "if (x->first < y->first) return -1;"),
    ("leaves_dropped_from_beam", "cand[n_cand++] = cur[t];\n                continue;", "continue;"),
    ("second_forest_ignored", "    if (ftau) {", "    if (0) {"),
    ("admission_strict", "(double)amax[c] >= tau", "(double)amax[c] > tau"),
    ("score_unscaled", "u = u * (1.0 / sqrt((double)d));", ""),
    ("prior_at_last_cell", "or_prior(p, head, i, f->first[node], (double)f->amax[node])",
     "or_prior(p, head, i, f->first[node] + 1, (double)f->amax[node])"),
]

# (name, text in fsb_plain.c, replacement)
PLAIN_MUTANTS = [
    ("plain_radius_term_dropped", "slack * sqrt(qq) * f->rho[node]", "0.0"),
    ("plain_radius_without_query_norm", "slack * sqrt(qq) * f->rho[node]",
     "slack * f->rho[node]"),
    ("plain_mean_not_divided", "mu[e] /= (double)width;", ";"),
    ("plain_radius_of_last_leaf", "if (acc > r2) r2 = acc;", "r2 = acc;"),
    ("plain_node_norm_of_first_leaf", "if (amax[c] > a_best) a_best = amax[c];",
     "if (t == 0) a_best = amax[c];"),
    ("plain_children_not_doubled", "e.index = 2 * cur[t].index + ch;",
     "e.index = cur[t].index + ch;"),
    ("plain_roots_unaligned", "index[cnt] = start >> l;", "index[cnt] = start;"),
    ("plain_ties_to_earlier_block", "return x->first > y->first ? -1 : 1;",
     "return x->first < y->first ? -1 : 1;"),
    ("plain_leaves_dropped_from_beam", "cand[n_cand++] = cur[t];\n                continue;",
     "continue;"),
    ("plain_second_forest_ignored", "    if (ftau)\n", "    if (0)\n"),
    ("plain_admission_strict", "amax[c] >= tau", "amax[c] > tau"),
    ("plain_score_unscaled", ") / sqrt((double)d);", ");"),
    ("plain_prior_at_next_cell", "or_prior(p, head, i, f->first[node], f->amax[node])",
     "or_prior(p, head, i, f->first[node] + 1, f->amax[node])"),
    ("plain_topk_off_by_one", "pl_cut(found, n_u, p->topk, &g)", "pl_cut(found, n_u, p->topk - 1, &g)"),
    ("plain_found_repeats", "dup |= found[r].first == found[t].first;", "dup |= 0;"),
]

CASES = [("fsb_oracle.c",) + m for m in MUTANTS] + [("fsb_plain.c",) + m for m in PLAIN_MUTANTS]


@pytest.mark.slow
@pytest.mark.parametrize("target,name,old,new", CASES, ids=[m[1] for m in CASES])
def test_fsb_pins_kill_mutant(tmp_path, target, name, old, new):
    for f in SOURCES + ("fs_oracle.h",):
        (tmp_path / f).write_text(open(os.path.join(ROOT, "oracle", f)).read())
    src = (tmp_path / target).read_text()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    (tmp_path / target).write_text(src.replace(old, new))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", str(lib), *[str(tmp_path / f) for f in SOURCES], "-lm",
                           "-lpthread"])
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_fsb_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
