"""The FS-B oracle's pins must catch plausible mistakes.

Each case plants one mistake in a copy of oracle/fsb_oracle.c (on the CPU
only), builds it with the unchanged fs_oracle.c, and runs
tests/test_oracle_fsb_pins.py against it in a subprocess; every mutant must
make at least one pin fail.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fsb_oracle.c")

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


@pytest.mark.slow
@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_fsb_pins_kill_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    c_path = tmp_path / "fsb_oracle.c"
    c_path.write_text(src.replace(old, new))
    for f in ("fs_oracle.c", "fs_oracle.h"):
        (tmp_path / f).write_text(open(os.path.join(ROOT, "oracle", f)).read())
    lib = tmp_path / "liboracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                           "-o", str(lib), str(tmp_path / "fs_oracle.c"), str(c_path), "-lm",
                           "-lpthread"])
    env = dict(os.environ, ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_fsb_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutant {name} survived the pins:\n{r.stdout[-2000:]}"
