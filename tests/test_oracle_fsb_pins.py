"""Pins of the FS-B oracle (FreeSolo paper summary, picx.dev page, section 3.4,
eqs. 10-11) against facts that do not come from the oracle itself.

- hand-worked searches on a four-cell forest (tests/golden/fsb_hand_cases.json);
- a beam wide enough to keep every node reduces the search to an exhaustive
  top-K, which must equal the FS-L oracle's eq. 7 selection over C_i (and,
  for the admitted forest, a brute-force top-K over {c in C_i : a_c >= tau});
- node statistics against their definitions computed by numpy;
- with slack 1, U_v bounds the eq. 7 score of every cell below v (Cauchy-
  Schwarz and the monotone erf), so the bound must hold for every node;
- the roots of a prefix are its binary decomposition;
- the fixed-order dot product against an exact rational sum.

Every pin except the last runs on both FS-B oracles: the fixed-order one
(fsb_oracle.c, float32 node statistics) and the plain fp64 one (fsb_plain.c).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import make_problem, with_prior

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fsb_hand_cases.json")


class _Plain:
    """The plain fp64 FS-B oracle with the FS-L oracle's other calls."""

    def __init__(self, orc):
        self.orc, self.plain = orc, orc.plain

    def __getattr__(self, name):
        if name in ("forest_build", "forest_roots", "node_score", "beam_row"):
            return getattr(self.plain, name)
        return getattr(self.orc, name)


@pytest.fixture(params=["fixed_order", "plain_fp64"])
def fsb(request, orc):
    return orc if request.param == "fixed_order" else _Plain(orc)


def _summaries(rng, n_cells, d):
    kbar = (rng.standard_normal((n_cells, d)) * 0.25).astype(np.float32)
    amax = (8.0 + 2.0 * rng.random(n_cells)).astype(np.float32)
    return kbar, amax


def test_golden_fsb(fsb):
    g = json.load(open(GOLDEN))
    d = 16
    kbar = np.zeros((4, d), np.float32)
    kbar[:, 0] = g["kbar0"]
    q = np.zeros(d, np.float32)
    q[0] = 1.0
    for case in g["cases"]:
        p = make_problem(head_dim=d, n_ctx=4 * 32, window=512, topk=case["topk"])
        am = np.array(case["tau_amax"] or [1, 1, 1, 1], np.float32)
        f0 = None if case.get("tau_only") else fsb.forest_build(kbar, am)
        ft = None if case["tau"] is None else fsb.forest_build(kbar, am, case["tau"])
        sel, sc = fsb.beam_row(p, 0, g["query_pos"], q, f0, ft, case["beam"], case["slack"])
        assert sel.tolist() == case["sel"], case["why"]
        np.testing.assert_allclose(sc, case["score"], rtol=0, atol=1e-12)


def test_golden_forest_stats(fsb):
    g = json.load(open(GOLDEN))
    kbar = np.zeros((4, 16), np.float32)
    kbar[:, 0] = g["kbar0"]
    f = fsb.forest_build(kbar, np.ones(4, np.float32))
    assert (f.m, f.n_levels) == (4, 3)
    assert f.mu[f.node(1, 0), 0] == 0 and f.rho[f.node(1, 0)] == 5
    assert f.mu[f.node(1, 1), 0] == 4 and f.rho[f.node(1, 1)] == 0
    assert f.mu[f.node(2, 0), 0] == 2 and f.rho[f.node(2, 0)] == 7


@pytest.mark.parametrize("n", [0, 1, 2, 3, 7, 8, 13, 64, 100, 1023])
def test_roots_are_binary_decomposition(fsb, n):
    kbar, amax = _summaries(np.random.default_rng(1), 1024, 16)
    f = fsb.forest_build(kbar, amax)
    roots = fsb.forest_roots(f, n)
    sizes = [1 << lv for lv, _ in roots]
    assert sizes == [1 << b for b in reversed(range(11)) if (n >> b) & 1]
    start = 0
    for lv, ix in roots:   # aligned, disjoint, covering [0, n) in order
        assert ix << lv == start
        start += 1 << lv
    assert start == n


def test_node_statistics_match_definitions(fsb):
    rng = np.random.default_rng(2)
    kbar, amax = _summaries(rng, 77, 64)
    for tau in (None, 9.0):
        f = fsb.forest_build(kbar, amax, tau)
        cells = np.arange(77) if tau is None else np.nonzero(amax >= tau)[0]
        assert f.m == len(cells) and f.cell_of[:f.m].tolist() == cells.tolist()
        assert f.prefix.tolist() == [int(np.sum(cells < n)) for n in range(78)]
        for lv in range(f.n_levels):
            for j in range(f.m >> lv):
                leaves = cells[j << lv:(j + 1) << lv]
                v = f.node(lv, j)
                mean = kbar[leaves].astype(np.float64).mean(axis=0)
                np.testing.assert_allclose(f.mu[v], mean, rtol=1e-6, atol=1e-7)
                dist = np.linalg.norm(kbar[leaves].astype(np.float64) - f.mu[v].astype(np.float64),
                                      axis=1).max()
                assert abs(f.rho[v] - dist) <= 1e-6 * max(dist, 1e-3)
                assert f.amax[v] == amax[leaves].max()
                assert f.first[v] == leaves[0]


def test_dot16_exact_for_integers(orc):
    rng = np.random.default_rng(3)
    for d in (16, 64, 128):
        a = rng.integers(-1000, 1000, d).astype(np.float32)
        b = rng.integers(-1000, 1000, d).astype(np.float32)
        assert orc.dot16(a, b) == float(sum(Fraction(int(x)) * int(y) for x, y in zip(a, b)))
        x = rng.standard_normal(d).astype(np.float32)
        y = rng.standard_normal(d).astype(np.float32)
        exact = sum(Fraction(float(u)) * Fraction(float(w)) for u, w in zip(x, y))
        assert abs(orc.dot16(x, y) - float(exact)) <= 1e-13 * float(sum(abs(Fraction(float(u)) * Fraction(float(w))) for u, w in zip(x, y)))


def _wide_problem(n_cells, d, topk, prior):
    p = make_problem(head_dim=d, n_ctx=n_cells * 32, window=512, topk=topk, heads=1)
    if prior:
        with_prior(p, [0.05], [900.0])
    return p


@pytest.mark.parametrize("prior", [False, True])
def test_exhaustive_beam_equals_eq7_topk(fsb, prior):
    """A beam that never drops a node finds every leaf, so S_i is eq. 7's top-K
    over C_i: compared with the FS-L oracle's selection (sets and scores)."""
    rng = np.random.default_rng(4)
    n_cells, d, topk = 150, 64, 12
    kbar, amax = _summaries(rng, n_cells, d)
    p = _wide_problem(n_cells, d, topk, prior)
    f0 = fsb.forest_build(kbar, amax)
    for _ in range(25):
        i = int(rng.integers(512, 512 + 32 * n_cells + 40))
        q = rng.standard_normal(d).astype(np.float32)
        n = fsb.n_candidates(p, i)
        sel, sc = fsb.beam_row(p, 0, i, q, f0, None, 2 * n_cells, 0.0)
        ref, _, ref_sc = fsb.select_row_at(p, 0, i, q, kbar.astype(np.float64),
                                           amax.astype(np.float64), np.arange(n, dtype=np.int32))
        assert sorted(sel.tolist()) == sorted(ref.tolist())
        np.testing.assert_allclose(sc, np.sort(ref_sc)[::-1][:len(sc)], rtol=1e-12, atol=1e-12)
        assert np.all(np.diff(sc) <= 0)


def test_exhaustive_admitted_forest_brute_force(fsb):
    rng = np.random.default_rng(5)
    n_cells, d, topk, tau = 120, 64, 10, 9.2
    kbar, amax = _summaries(rng, n_cells, d)
    p = _wide_problem(n_cells, d, topk, False)
    ft = fsb.forest_build(kbar, amax, tau)
    f0 = fsb.forest_build(kbar, amax)
    for _ in range(20):
        i = int(rng.integers(512, 512 + 32 * n_cells))
        q = rng.standard_normal(d).astype(np.float32)
        n = fsb.n_candidates(p, i)
        scores = kbar[:n].astype(np.float64) @ q.astype(np.float64) / 8.0
        adm = np.nonzero(amax[:n] >= tau)[0]
        sel, _ = fsb.beam_row(p, 0, i, q, None, ft, 2 * n_cells, 0.0)
        assert sorted(sel.tolist()) == sorted(adm[np.argsort(-scores[adm])][:topk].tolist())
        # both forests, exhaustive: the admitted cells are a subset, so eq. 7 over C_i
        sel2, _ = fsb.beam_row(p, 0, i, q, f0, ft, 2 * n_cells, 0.0)
        assert sorted(sel2.tolist()) == sorted(np.argsort(-scores)[:topk].tolist())


@pytest.mark.parametrize("prior", [False, True])
def test_slack_one_bounds_every_leaf(fsb, prior):
    """Eq. 11 with c = 1: q.mu + |q| rho >= q.kbar_c (Cauchy-Schwarz) and
    A_v g(i - p_min) >= a_c g(i - p_c) (erf increasing, g >= 0 on C_i)."""
    rng = np.random.default_rng(6)
    n_cells, d = 64, 64
    kbar, amax = _summaries(rng, n_cells, d)
    p = _wide_problem(n_cells, d, 8, prior)
    f = fsb.forest_build(kbar, amax)
    i = 512 + 32 * n_cells
    for _ in range(5):
        q = rng.standard_normal(d).astype(np.float32)
        leaf = [fsb.node_score(p, 0, i, q, f, 0, j, 1.0) for j in range(f.m)]
        for lv in range(1, f.n_levels):
            for j in range(f.m >> lv):
                u = fsb.node_score(p, 0, i, q, f, lv, j, 1.0)
                assert u >= max(leaf[j << lv:(j + 1) << lv]) - 1e-12
        # a leaf's U is eq. 7's score
        _, _, ref = fsb.select_row_at(p, 0, i, q, kbar.astype(np.float64),
                                      amax.astype(np.float64), np.arange(n_cells, dtype=np.int32))
        np.testing.assert_allclose(leaf, ref, rtol=1e-12, atol=1e-12)


def test_empty_and_narrow(fsb):
    rng = np.random.default_rng(7)
    kbar, amax = _summaries(rng, 40, 64)
    p = _wide_problem(40, 64, 8, False)
    f0 = fsb.forest_build(kbar, amax)
    q = rng.standard_normal(64).astype(np.float32)
    sel, _ = fsb.beam_row(p, 0, 100, q, f0, None, 8, 1.0)        # i < w: C_i empty
    assert len(sel) == 0
    sel, _ = fsb.beam_row(p, 0, 512 + 32 * 3, q, f0, None, 8, 1.0)   # n_i = 3 < K
    assert sorted(sel.tolist()) == [0, 1, 2]
    ft = fsb.forest_build(kbar, amax, 100.0)                     # nothing admitted
    assert ft.m == 0
    sel, _ = fsb.beam_row(p, 0, 512 + 32 * 40, q, None, ft, 8, 1.0)
    assert len(sel) == 0


def test_search_effort_closed_form(fsb):
    """Nodes scored by one forest's search: the roots, plus two per inner node of
    each step's beam.  With a beam that never drops a node (width >= leaves), every
    node of the covering trees is scored exactly once: 2 * 2^l - 1 per root of
    level l."""
    rng = np.random.default_rng(8)
    n_cells, d = 90, 64
    kbar, amax = _summaries(rng, n_cells, d)
    p = _wide_problem(n_cells, d, 8, False)
    f0 = fsb.forest_build(kbar, amax)
    for n in (1, 5, 16, 37, 90):
        i = 512 + 32 * n
        q = rng.standard_normal(d).astype(np.float32)
        *_, e = fsb.beam_row(p, 0, i, q, f0, None, 2 * n_cells, 0.0, effort=True)
        assert e == sum(2 * (1 << lv) - 1 for lv, _ in fsb.forest_roots(f0, n))
        # a beam of width 1 scores the roots, then two children per level below the
        # best root: at most roots + 2 * (its level)
        *_, e1 = fsb.beam_row(p, 0, i, q, f0, None, 1, 0.0, effort=True)
        roots = fsb.forest_roots(f0, n)
        assert len(roots) <= e1 <= len(roots) + 2 * max(lv for lv, _ in roots)


@pytest.mark.parametrize("prior", [False, True])
def test_plain_and_fixed_order_agree_where_decided(orc, prior):
    """The two FS-B oracles round differently (fp64 from fp64 summaries against a
    fixed order on float32 statistics), so they may part only at a near-tie
    decision: every row whose plain-oracle gap is at least 1e-5 selects the same
    cells with the same search effort."""
    rng = np.random.default_rng(9)
    n_cells, d, topk = 300, 64, 8
    kb64 = rng.standard_normal((n_cells, d)) * 0.2
    am64 = 8.0 + 2.0 * rng.random(n_cells)
    p = _wide_problem(n_cells, d, topk, prior)
    tau = float(np.float32(np.quantile(am64, 0.6)))
    pf0, pft = orc.plain.forest_build(kb64, am64), orc.plain.forest_build(kb64, am64, tau)
    kb32, am32 = kb64.astype(np.float32), am64.astype(np.float32)
    f0, ft = orc.forest_build(kb32, am32), orc.forest_build(kb32, am32, tau)
    qs = rng.standard_normal((400, d)).astype(np.float32)
    p.q_pos0 = 512 + 32 * n_cells - 400
    ref = orc.plain.beam_rows(p, 0, qs, np.arange(400), pf0, pft, 6, 1.0, 4)
    decided = 0
    for t in range(400):
        sel, _, eff = orc.beam_row(p, 0, p.q_pos0 + t, qs[t], f0, ft, 6, 1.0, effort=True)
        if ref["gap"][t] < 1e-5:
            continue
        decided += 1
        assert sorted(sel.tolist()) == sorted(ref["sel"][t, :ref["n_sel"][t]].tolist()), t
        assert eff == ref["effort"][t], t
    assert decided >= 390


def test_found_cells_of_an_exhaustive_search(orc):
    """A beam as wide as the leaves keeps every node, so the plain oracle's found
    cells are all of C_i (forest 0), the admitted cells of C_i (forest tau), and
    with both forests C_i again: the admitted cells come twice and are kept once."""
    rng = np.random.default_rng(10)
    n_cells, d, tau = 60, 64, 9.0
    kbar, amax = _summaries(rng, n_cells, d)
    p = _wide_problem(n_cells, d, 8, True)
    f0 = orc.plain.forest_build(kbar, amax)
    ft = orc.plain.forest_build(kbar, amax, tau)
    for _ in range(12):
        i = int(rng.integers(512, 512 + 32 * n_cells + 40))
        q = rng.standard_normal(d).astype(np.float32)
        n = orc.n_candidates(p, i)
        cells, _ = orc.plain.beam_found(p, 0, i, q, f0, None, 64, 0.0)
        assert sorted(cells.tolist()) == list(range(n))
        cells, _ = orc.plain.beam_found(p, 0, i, q, None, ft, 64, 0.0)
        assert sorted(cells.tolist()) == np.nonzero(amax[:n] >= tau)[0].tolist()
        cells, _ = orc.plain.beam_found(p, 0, i, q, f0, ft, 64, 0.0)
        assert sorted(cells.tolist()) == list(range(n))


@pytest.mark.parametrize("prior", [False, True])
def test_rerank_of_found_cells_with_constant_keys(orc, prior):
    """When a cell's s keys all equal its mean key, eq. 12's score is eq. 7's plus
    ln s (a log-sum-exp of s equal logits), so reranking the cells a search
    found picks the same cells as the search's own eq. 7 top-K."""
    rng = np.random.default_rng(11)
    n_cells, d, topk, s = 200, 64, 8, 32
    kbar, amax = _summaries(rng, n_cells, d)
    k_head = np.repeat(kbar, s, axis=0)
    p = _wide_problem(n_cells, d, topk, prior)
    f0 = orc.plain.forest_build(kbar, amax)
    ft = orc.plain.forest_build(kbar, amax, 9.3)
    am64 = amax.astype(np.float64)
    for _ in range(20):
        i = int(rng.integers(512 + 32 * 20, 512 + 32 * n_cells))
        q = rng.standard_normal(d).astype(np.float32)
        cells, gap = orc.plain.beam_found(p, 0, i, q, f0, ft, 6, 1.0)
        sel, sc = orc.plain.beam_row(p, 0, i, q, f0, ft, 6, 1.0)
        rr, _, rr_sc = orc.rerank_row(p, 0, i, q, k_head, am64, cells)
        assert sorted(rr.tolist()) == sorted(sel.tolist())
        _, _, u = orc.select_row_at(p, 0, i, q, kbar.astype(np.float64), am64, cells)
        np.testing.assert_allclose(rr_sc, u + math.log(s), rtol=1e-12, atol=1e-12)
