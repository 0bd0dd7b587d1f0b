"""ctypes wrapper of the fp64 CPU oracle (fs_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the CPU
baseline leg of the benchmark.  The product path never imports it.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
SRC_PATH = os.path.join(_HERE, "fs_oracle.c")
FSB_SRC_PATH = os.path.join(_HERE, "fsb_oracle.c")
FSB_PLAIN_SRC_PATH = os.path.join(_HERE, "fsb_plain.c")


def build(force: bool = True) -> str:
    """Compile fs_oracle.c, fsb_oracle.c and fsb_plain.c with gcc into liboracle.so
    (plain -O2, no fast-math, no fp contraction)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fPIC", "-shared",
                               "-Wall", "-o", tmp, SRC_PATH, FSB_SRC_PATH, FSB_PLAIN_SRC_PATH,
                               "-lm", "-lpthread"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


class Problem(C.Structure):
    _fields_ = [("batch", C.c_int), ("heads", C.c_int), ("head_dim", C.c_int),
                ("n_ctx", C.c_int), ("n_q", C.c_int), ("q_pos0", C.c_int),
                ("cell", C.c_int), ("window", C.c_int), ("topk", C.c_int),
                ("budget", C.c_int), ("n_recent", C.c_int),
                ("rope_base", C.c_double), ("rms_eps", C.c_double),
                ("pos_offset", C.c_longlong),
                ("prior_lambda", C.c_void_p), ("prior_sigma", C.c_void_p)]


def with_prior(p: Problem, lam, sigma) -> Problem:
    """Attach per-head eq. 7 prior arrays (kept alive on the Problem object)."""
    p._lam = np.ascontiguousarray(lam, dtype=np.float64)
    p._sig = np.ascontiguousarray(sigma, dtype=np.float64)
    assert p._lam.shape == (p.heads,) and p._sig.shape == (p.heads,)
    p.prior_lambda = p._lam.ctypes.data
    p.prior_sigma = p._sig.ctypes.data
    return p


def problem_from(wl, **kw) -> Problem:
    """Oracle problem for a synth.Workload, with optional field overrides."""
    f = dict(batch=wl.batch, heads=wl.heads, head_dim=wl.head_dim, n_ctx=wl.n_ctx,
             n_q=wl.n_q, q_pos0=wl.q_pos0, cell=wl.cell, window=wl.window, topk=wl.topk,
             budget=wl.budget, n_recent=wl.n_recent, rope_base=wl.rope_base,
             rms_eps=wl.rms_eps, pos_offset=0)
    f.update(kw)
    p = Problem(**f)
    lam, sig = getattr(wl, "prior_arrays", lambda: (None, None))()
    if lam is not None:
        with_prior(p, lam, sig)
    return p


def make_problem(**kw) -> Problem:
    f = dict(batch=1, heads=1, head_dim=64, n_ctx=0, n_q=0, q_pos0=0, cell=32, window=512,
             topk=8, budget=-1, n_recent=0, rope_base=10000.0, rms_eps=1e-6, pos_offset=0)
    f.update(kw)
    return Problem(**f)


_F32P = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_F64P = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_I32P = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")


def _f32(x):
    return np.ascontiguousarray(x, dtype=np.float32)


def _f64(x):
    return np.ascontiguousarray(x, dtype=np.float64)


def _i32(x):
    return np.ascontiguousarray(x, dtype=np.int32)


class _ForestStruct(C.Structure):
    _fields_ = [("n_cells", C.c_int), ("head_dim", C.c_int), ("m", C.c_int),
                ("n_levels", C.c_int), ("level_start", C.c_int * 32),
                ("cell_of", C.c_void_p), ("prefix", C.c_void_p), ("first", C.c_void_p),
                ("amax", C.c_void_p), ("rho", C.c_void_p), ("mu", C.c_void_p)]


class Forest:
    """One FS-B causal forest of one head (section 3.4), with numpy views of its
    node arrays: node (l, j) is row level_start[l] + j."""

    def __init__(self, n_cells: int, d: int):
        n = max(n_cells, 1)
        self.cell_of = np.zeros(n, np.int32)
        self.prefix = np.zeros(n + 1, np.int32)
        self.first = np.zeros(2 * n, np.int32)
        self.amax = np.zeros(2 * n, np.float32)
        self.rho = np.zeros(2 * n, np.float32)
        self.mu = np.zeros((2 * n, d), np.float32)
        self.s = _ForestStruct(n_cells, d, 0, 0, (C.c_int * 32)(),
                               self.cell_of.ctypes.data, self.prefix.ctypes.data,
                               self.first.ctypes.data, self.amax.ctypes.data,
                               self.rho.ctypes.data, self.mu.ctypes.data)

    @property
    def m(self) -> int:
        return self.s.m

    @property
    def n_levels(self) -> int:
        return self.s.n_levels

    def node(self, level: int, index: int) -> int:
        return self.s.level_start[level] + index


class _Forest64Struct(C.Structure):
    _fields_ = [("n_cells", C.c_int), ("head_dim", C.c_int), ("m", C.c_int),
                ("n_levels", C.c_int), ("level_start", C.c_int * 32),
                ("cell_of", C.c_void_p), ("prefix", C.c_void_p), ("first", C.c_void_p),
                ("amax", C.c_void_p), ("rho", C.c_void_p), ("mu", C.c_void_p)]


class Forest64(Forest):
    """A forest of the plain fp64 FS-B oracle (fsb_plain.c): node statistics in
    float64, from float64 cell summaries."""

    def __init__(self, n_cells: int, d: int):
        n = max(n_cells, 1)
        self.cell_of = np.zeros(n, np.int32)
        self.prefix = np.zeros(n + 1, np.int32)
        self.first = np.zeros(2 * n, np.int32)
        self.amax = np.zeros(2 * n, np.float64)
        self.rho = np.zeros(2 * n, np.float64)
        self.mu = np.zeros((2 * n, d), np.float64)
        self.s = _Forest64Struct(n_cells, d, 0, 0, (C.c_int * 32)(),
                                 self.cell_of.ctypes.data, self.prefix.ctypes.data,
                                 self.first.ctypes.data, self.amax.ctypes.data,
                                 self.rho.ctypes.data, self.mu.ctypes.data)


class PlainFsb:
    """The plain fp64 FS-B oracle (fsb_plain.c) behind the interface of the
    fixed-order one: forest_build, forest_roots, node_score, beam_row, plus
    beam_rows for many rows with each row's decision gap."""

    def __init__(self, orc: "Oracle"):
        self.orc, self.L = orc, orc.L

    def forest_build(self, kbar, amax, tau: float | None = None) -> Forest64:
        kbar, amax = _f64(kbar), _f64(amax)
        n_cells, d = kbar.shape
        f = Forest64(n_cells, d)
        self.L.or_forest64_build(kbar if n_cells else np.zeros((1, d)),
                                 amax if n_cells else np.zeros(1), n_cells, d,
                                 0 if tau is None else 1, 0.0 if tau is None else float(tau),
                                 C.byref(f.s))
        return f

    def forest_roots(self, f: Forest64, n_leaves: int):
        lv = np.zeros(32, np.int32)
        ix = np.zeros(32, np.int32)
        cnt = self.L.or_forest64_roots(C.byref(f.s), int(n_leaves), lv, ix)
        return list(zip(lv[:cnt].tolist(), ix[:cnt].tolist()))

    def node_score(self, p: Problem, head: int, i: int, q_row, f: Forest64, level: int,
                   index: int, slack: float) -> float:
        return self.L.or_node64_score(C.byref(p), int(head), int(i), _f32(q_row), C.byref(f.s),
                                      int(level), int(index), float(slack))

    def beam_row(self, p: Problem, head: int, i: int, q_row, f0, ftau, beam: int, slack: float,
                 effort: bool = False, gap: bool = False):
        sel = np.zeros(max(p.topk, 1), np.int32)
        sc = np.zeros(max(p.topk, 1), np.float64)
        n_scored, g = C.c_int(), C.c_double()
        cnt = self.L.or_beam64_row(C.byref(p), int(head), int(i), _f32(q_row),
                                   None if f0 is None else C.addressof(f0.s),
                                   None if ftau is None else C.addressof(ftau.s),
                                   int(beam), float(slack), sel, sc, C.byref(n_scored),
                                   C.byref(g))
        out = (sel[:cnt].copy(), sc[:cnt].copy())
        if effort:
            out += (n_scored.value,)
        if gap:
            out += (g.value,)
        return out

    def beam_found(self, p: Problem, head: int, i: int, q_row, f0, ftau, beam: int,
                   slack: float):
        """The cells the two searches end with (no repeats) and the searches' gap."""
        cells = np.zeros(2 * beam + 2, np.int32)
        n_scored, g = C.c_int(), C.c_double()
        cnt = self.L.or_beam64_found(C.byref(p), int(head), int(i), _f32(q_row),
                                     None if f0 is None else C.addressof(f0.s),
                                     None if ftau is None else C.addressof(ftau.s), int(beam),
                                     float(slack), cells, C.byref(n_scored), C.byref(g))
        return cells[:cnt].copy(), g.value

    def beam_rows(self, p: Problem, head: int, q_head, rows, f0, ftau, beam: int, slack: float,
                  nthreads: int | None = None) -> dict:
        """S_i of query rows `rows` (indices into q_head, positions q_pos0 + t):
        sel / score [n, K] descending, -1 / 0 padded; n_sel, effort, gap [n]."""
        rows = _i32(rows)
        n, K = len(rows), p.topk
        sel = np.empty((max(n, 1), K), np.int32)
        sc = np.empty((max(n, 1), K), np.float64)
        n_sel = np.empty(max(n, 1), np.int32)
        eff = np.empty(max(n, 1), np.int32)
        gap = np.empty(max(n, 1), np.float64)
        self.L.or_beam64_rows(C.byref(p), int(head), _f32(q_head), rows, n,
                              None if f0 is None else C.addressof(f0.s),
                              None if ftau is None else C.addressof(ftau.s), int(beam),
                              float(slack), sel, sc, n_sel, eff, gap,
                              int(nthreads or os.cpu_count() or 1))
        return dict(sel=sel[:n], score=sc[:n], n_sel=n_sel[:n], effort=eff[:n], gap=gap[:n])


class Oracle:
    def __init__(self, path: str | None = None):
        path = path or LIB_PATH
        if not os.path.exists(path):
            build()
        L = C.CDLL(path)
        P = C.POINTER(Problem)
        L.or_rope.argtypes = [P, _F32P, C.c_longlong, _F64P]
        L.or_n_candidates.argtypes = [P, C.c_longlong]
        L.or_n_candidates.restype = C.c_int
        L.or_cell_summaries_head.argtypes = [P, _F32P, _F64P, _F64P]
        L.or_prune_row.argtypes = [P, _F64P, C.c_int, _I32P, C.POINTER(C.c_double)]
        L.or_prune_row.restype = C.c_int
        L.or_select_row.argtypes = [P, _F32P, _F64P, _I32P, C.c_int, _I32P,
                                    C.POINTER(C.c_double), C.c_void_p]
        L.or_select_row.restype = C.c_int
        L.or_select_row_at.argtypes = [P, C.c_int, C.c_longlong, _F32P, _F64P, C.c_void_p,
                                       _I32P, C.c_int, _I32P, C.POINTER(C.c_double), C.c_void_p]
        L.or_select_row_at.restype = C.c_int
        L.or_rerank_row.argtypes = [P, C.c_int, C.c_longlong, _F32P, _F32P, C.c_void_p,
                                    _I32P, C.c_int, _I32P, C.POINTER(C.c_double), C.c_void_p]
        L.or_rerank_row.restype = C.c_int
        L.or_prior.argtypes = [P, C.c_int, C.c_longlong, C.c_int, C.c_double]
        L.or_prior.restype = C.c_double
        L.or_window_row.argtypes = [P, _F32P, _F32P, _F32P, C.c_longlong, _F64P]
        L.or_sparse_row.argtypes = [P, _F32P, _F32P, _F32P, _I32P, C.c_int, _F64P]
        vp = C.c_void_p
        L.or_forward_rows.argtypes = [P, _F32P, _F32P, _F32P, _F64P, _F64P, C.c_double,
                                      _I32P, C.c_int, vp, vp, C.c_int, vp, vp,
                                      _F64P, _F64P, _F64P, _I32P, _I32P, _F64P, _F64P, C.c_int,
                                      C.c_int]
        L.or_forward.argtypes = [P, _F32P, _F32P, _F32P, _F32P, _F64P, _F64P, _F64P,
                                 _I32P, _I32P, _F64P, _F64P, C.c_int]
        FP = C.POINTER(_ForestStruct)
        L.or_dot16.argtypes = [_F32P, _F32P, C.c_int]
        L.or_dot16.restype = C.c_double
        L.or_forest_build.argtypes = [_F32P, _F32P, C.c_int, C.c_int, C.c_int, C.c_double, FP]
        L.or_forest_build.restype = C.c_int
        L.or_forest_roots.argtypes = [FP, C.c_int, _I32P, _I32P]
        L.or_forest_roots.restype = C.c_int
        L.or_node_score.argtypes = [P, C.c_int, C.c_longlong, _F32P, C.c_double, FP, C.c_int,
                                    C.c_int, C.c_double]
        L.or_node_score.restype = C.c_double
        L.or_beam_row.argtypes = [P, C.c_int, C.c_longlong, _F32P, C.c_void_p, C.c_void_p,
                                  C.c_int, C.c_double, _I32P, _F64P, C.POINTER(C.c_int)]
        L.or_beam_row.restype = C.c_int
        F64 = C.POINTER(_Forest64Struct)
        L.or_forest64_build.argtypes = [_F64P, _F64P, C.c_int, C.c_int, C.c_int, C.c_double, F64]
        L.or_forest64_build.restype = C.c_int
        L.or_forest64_roots.argtypes = [F64, C.c_int, _I32P, _I32P]
        L.or_forest64_roots.restype = C.c_int
        L.or_node64_score.argtypes = [P, C.c_int, C.c_longlong, _F32P, F64, C.c_int, C.c_int,
                                      C.c_double]
        L.or_node64_score.restype = C.c_double
        L.or_beam64_row.argtypes = [P, C.c_int, C.c_longlong, _F32P, C.c_void_p, C.c_void_p,
                                    C.c_int, C.c_double, _I32P, _F64P, C.POINTER(C.c_int),
                                    C.POINTER(C.c_double)]
        L.or_beam64_row.restype = C.c_int
        L.or_beam64_found.argtypes = [P, C.c_int, C.c_longlong, _F32P, C.c_void_p, C.c_void_p,
                                      C.c_int, C.c_double, _I32P, C.POINTER(C.c_int),
                                      C.POINTER(C.c_double)]
        L.or_beam64_found.restype = C.c_int
        L.or_beam64_rows.argtypes = [P, C.c_int, _F32P, _I32P, C.c_int, C.c_void_p, C.c_void_p,
                                     C.c_int, C.c_double, _I32P, _F64P, _I32P, _I32P, _F64P,
                                     C.c_int]
        L.or_beam64_rows.restype = C.c_int
        self.L = L
        self.plain = PlainFsb(self)

    # -- FS-B (section 3.4) ---------------------------------------------------
    def dot16(self, a, b) -> float:
        a, b = _f32(a), _f32(b)
        return self.L.or_dot16(a, b, a.shape[0])

    def forest_build(self, kbar, amax, tau: float | None = None) -> Forest:
        """Forest over one head's fp32 summaries: every cell (tau None, A^0) or the
        cells with amax >= tau (A^tau, eq. 10)."""
        kbar, amax = _f32(kbar), _f32(amax)
        n_cells, d = kbar.shape
        f = Forest(n_cells, d)
        self.L.or_forest_build(kbar if n_cells else np.zeros((1, d), np.float32),
                               amax if n_cells else np.zeros(1, np.float32), n_cells, d,
                               0 if tau is None else 1, 0.0 if tau is None else float(tau),
                               C.byref(f.s))
        return f

    def forest_roots(self, f: Forest, n_leaves: int):
        lv = np.zeros(32, np.int32)
        ix = np.zeros(32, np.int32)
        cnt = self.L.or_forest_roots(C.byref(f.s), int(n_leaves), lv, ix)
        return list(zip(lv[:cnt].tolist(), ix[:cnt].tolist()))

    def node_score(self, p: Problem, head: int, i: int, q_row, f: Forest, level: int,
                   index: int, slack: float) -> float:
        q = _f32(q_row)
        qn = float(np.sqrt(self.dot16(q, q)))
        return self.L.or_node_score(C.byref(p), int(head), int(i), q, qn, C.byref(f.s),
                                    int(level), int(index), float(slack))

    def beam_row(self, p: Problem, head: int, i: int, q_row, f0: Forest | None,
                 ftau: Forest | None, beam: int, slack: float, effort: bool = False):
        """S_i of the query at position i by beam search (eqs. 10-11), with its eq. 7
        scores, in descending (score, cell) order.  With effort=True also returns
        the number of node scores the searches computed."""
        sel = np.zeros(max(p.topk, 1), np.int32)
        sc = np.zeros(max(p.topk, 1), np.float64)
        n_scored = C.c_int()
        cnt = self.L.or_beam_row(C.byref(p), int(head), int(i), _f32(q_row),
                                 None if f0 is None else C.addressof(f0.s),
                                 None if ftau is None else C.addressof(ftau.s),
                                 int(beam), float(slack), sel, sc, C.byref(n_scored))
        if effort:
            return sel[:cnt].copy(), sc[:cnt].copy(), n_scored.value
        return sel[:cnt].copy(), sc[:cnt].copy()

    # -- single steps ------------------------------------------------------
    def rope(self, p: Problem, x, pos: int) -> np.ndarray:
        out = np.empty(p.head_dim, np.float64)
        self.L.or_rope(C.byref(p), _f32(x), int(pos), out)
        return out

    def n_candidates(self, p: Problem, i: int) -> int:
        return self.L.or_n_candidates(C.byref(p), int(i))

    def cell_summaries_head(self, p: Problem, k_head):
        C_ = p.n_ctx // p.cell
        kbar = np.empty((max(C_, 1), p.head_dim), np.float64)
        amax = np.empty(max(C_, 1), np.float64)
        self.L.or_cell_summaries_head(C.byref(p), _f32(k_head), kbar, amax)
        return kbar[:C_], amax[:C_]

    def prune_row(self, p: Problem, amax, n: int):
        keep = np.empty(max(n, 1), np.int32)
        gap = C.c_double()
        cnt = self.L.or_prune_row(C.byref(p), _f64(amax), int(n), keep, C.byref(gap))
        return keep[:cnt].copy(), gap.value

    def select_row(self, p: Problem, q_row, kbar, cand):
        cand = _i32(cand)
        sel = np.empty(max(len(cand), 1), np.int32)
        scores = np.empty(max(len(cand), 1), np.float64)
        gap = C.c_double()
        cnt = self.L.or_select_row(C.byref(p), _f32(q_row), _f64(kbar), cand, len(cand), sel,
                                   C.byref(gap), scores.ctypes.data)
        return sel[:cnt].copy(), gap.value, scores[:len(cand)].copy()

    def select_row_at(self, p: Problem, head: int, i: int, q_row, kbar, amax, cand):
        """Eq. 7 scores with the problem's position prior (if any) for the query at
        position i of head `head`."""
        cand = _i32(cand)
        sel = np.empty(max(len(cand), 1), np.int32)
        scores = np.empty(max(len(cand), 1), np.float64)
        gap = C.c_double()
        am = None if amax is None else _f64(amax)
        cnt = self.L.or_select_row_at(C.byref(p), int(head), int(i), _f32(q_row), _f64(kbar),
                                      None if am is None else am.ctypes.data, cand, len(cand),
                                      sel, C.byref(gap), scores.ctypes.data)
        return sel[:cnt].copy(), gap.value, scores[:len(cand)].copy()

    def rerank_row(self, p: Problem, head: int, i: int, q_row, k_head, amax, cand):
        """Eq. 12 scores (log-sum-exp of the cell's token logits + the prior, if
        any) and the top-K of the query at position i of head `head`."""
        cand = _i32(cand)
        sel = np.empty(max(len(cand), 1), np.int32)
        scores = np.empty(max(len(cand), 1), np.float64)
        gap = C.c_double()
        am = None if amax is None else _f64(amax)
        cnt = self.L.or_rerank_row(C.byref(p), int(head), int(i), _f32(q_row), _f32(k_head),
                                   None if am is None else am.ctypes.data, cand, len(cand), sel,
                                   C.byref(gap), scores.ctypes.data)
        return sel[:cnt].copy(), gap.value, scores[:len(cand)].copy()

    def prior(self, p: Problem, head: int, i: int, c: int, a_c: float) -> float:
        return self.L.or_prior(C.byref(p), int(head), int(i), int(c), float(a_c))

    def window_row(self, p: Problem, q_row, k_head, v_head, i: int) -> np.ndarray:
        out = np.empty(p.head_dim, np.float64)
        self.L.or_window_row(C.byref(p), _f32(q_row), _f32(k_head), _f32(v_head), int(i), out)
        return out

    def sparse_row(self, p: Problem, q_row, k_head, v_head, sel) -> np.ndarray:
        n_sel = len(sel)
        arr = _i32(sel) if n_sel else np.zeros(1, np.int32)
        out = np.empty(p.head_dim, np.float64)
        self.L.or_sparse_row(C.byref(p), _f32(q_row), _f32(k_head), _f32(v_head), arr, n_sel,
                             out)
        return out

    # -- composed -------------------------------------------------------------
    def forward_rows(self, p: Problem, q_head, k_head, v_head, kbar, amax, alpha, rows,
                     keep_ovr=None, sel_ovr=None, nthreads: int | None = None,
                     head: int = 0) -> dict:
        """Forward of one head for query rows ``rows`` (indices into q_head).

        keep_ovr / sel_ovr: optional lists (one entry per row, None = no
        override) of the retained / selected cell sets to use instead of the
        oracle's own."""
        rows = _i32(rows)
        n = len(rows)
        d, K = p.head_dim, p.topk
        nthreads = nthreads or os.cpu_count() or 1
        keep_p = keep_n_p = sel_p = sel_n_p = None
        keep_w = 0
        hold = []
        if keep_ovr is not None:
            keep_w = max([len(x) for x in keep_ovr if x is not None] + [1])
            ka = np.full((n, keep_w), -1, np.int32)
            kn = np.full(n, -1, np.int32)
            for r, x in enumerate(keep_ovr):
                if x is not None:
                    ka[r, :len(x)] = x
                    kn[r] = len(x)
            hold += [ka, kn]
            keep_p, keep_n_p = ka.ctypes.data, kn.ctypes.data
        if sel_ovr is not None:
            sa = np.full((n, K), -1, np.int32)
            sn = np.full(n, -1, np.int32)
            for r, x in enumerate(sel_ovr):
                if x is not None:
                    sa[r, :len(x)] = x
                    sn[r] = len(x)
            hold += [sa, sn]
            sel_p, sel_n_p = sa.ctypes.data, sn.ctypes.data
        o = np.empty((n, d)); o_sr = np.empty((n, d)); o_lr = np.empty((n, d))
        sel = np.empty((n, K), np.int32); n_sel = np.empty(n, np.int32)
        sg = np.empty(n); kg = np.empty(n)
        kbar_c = _f64(kbar) if len(kbar) else np.zeros((1, d))
        amax_c = _f64(amax) if len(amax) else np.zeros(1)
        self.L.or_forward_rows(C.byref(p), _f32(q_head), _f32(k_head), _f32(v_head), kbar_c,
                               amax_c, float(alpha), rows, n, keep_p, keep_n_p, keep_w, sel_p,
                               sel_n_p, o, o_sr, o_lr, sel, n_sel, sg, kg, int(nthreads),
                               int(head))
        return dict(o=o, o_sr=o_sr, o_lr=o_lr, sel=sel, n_sel=n_sel, sel_gap=sg, keep_gap=kg)

    def forward(self, p: Problem, q, k, v, alpha, nthreads: int | None = None) -> dict:
        B, H, nq, d, K = p.batch, p.heads, p.n_q, p.head_dim, p.topk
        nthreads = nthreads or os.cpu_count() or 1
        o = np.empty((B, H, nq, d)); o_sr = np.empty_like(o); o_lr = np.empty_like(o)
        sel = np.empty((B, H, nq, K), np.int32); n_sel = np.empty((B, H, nq), np.int32)
        sg = np.empty((B, H, nq)); kg = np.empty((B, H, nq))
        self.L.or_forward(C.byref(p), _f32(q), _f32(k), _f32(v), _f32(alpha), o, o_sr, o_lr,
                          sel, n_sel, sg, kg, int(nthreads))
        return dict(o=o, o_sr=o_sr, o_lr=o_lr, sel=sel, n_sel=n_sel, sel_gap=sg, keep_gap=kg)
