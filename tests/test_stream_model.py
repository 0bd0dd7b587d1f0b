"""The bounded-memory property the streaming state rests on (FreeSolo summary,
"Bounded memory" under Practical Implications, with eq. 8).

A fixed number of cell slots, filled as cells become candidates and released
when a cell leaves both Recent_W and TopP, reproduces eq. 8's keep set
A = Recent_W(C) u TopP(a) for every prefix: TopP over [0, n + 1) only ever takes
cell n into TopP over [0, n), so a cell once dropped is never needed again.

`StreamModel` is the streaming state's update in plain Python, step by step as
the device code does it (the newest cell wins a tie on a_c; TopP kept in
ascending cell order; a released slot returns to the free list one step later,
because earlier queries of the same step may still read it).  Its keep sets are
compared with the oracle's eq. 8 rows over the whole prefix, and its slot use
with the bound W + P + ceil(B / s) + 2 the state is sized for.
"""
import numpy as np
import pytest

import oracle


def n_cand(i, w, s):
    return 0 if i < w else (i - w) // s


class StreamModel:
    def __init__(self, W, P, s, w, max_new):
        self.W, self.P, self.s, self.w = W, P, s, w
        self.M = W + P + (max_new + s - 1) // s + 2
        self.free = list(range(self.M - 1, -1, -1))
        self.pend = []
        self.topp = []            # (a, c, slot), ascending c
        self.recent = {}          # c % W -> slot
        self.slot_cell = {}
        self.pos = 0

    def step(self, amax, n_new):
        """Append n_new tokens; return {n: [(cell, slot), ...]} for the step's counts."""
        W, P, s, w = self.W, self.P, self.s, self.w
        self.free += self.pend
        self.pend = []
        for sl in self.free:
            self.slot_cell.pop(sl, None)
        pos0 = self.pos
        n_start = 0 if pos0 == 0 else n_cand(pos0 - 1, w, s)
        n_row0, n_end = n_cand(pos0, w, s), n_cand(pos0 + n_new - 1, w, s)
        rows = {}

        def emit(n):
            pre = [(c, sl) for (_, c, sl) in self.topp if c < n - W]
            rec = [(c, self.recent[c % W]) for c in range(max(0, n - W), n)]
            rows[n] = pre + rec

        if n_row0 == n_start:
            emit(n_start)
        for c in range(n_start, n_end):
            a = float(amax[c])
            enter, ev = len(self.topp) < P, -1
            if not enter and P > 0:
                j = min(range(len(self.topp)), key=lambda t: (self.topp[t][0], self.topp[t][1]))
                enter = a >= self.topp[j][0]
                ev = j if enter else -1
            ce, se = (self.topp[ev][1], self.topp[ev][2]) if ev >= 0 else (-1, -1)
            cr = c - W if W > 0 and c - W >= 0 else -1
            sr = self.recent[cr % W] if cr >= 0 else -1
            retained = enter or W > 0
            assert not retained or self.free, "slot pool exhausted"
            slot = self.free.pop() if retained else -1
            in_topp = {t[2] for t in self.topp}
            drop_e = ev >= 0 and ce <= c - W
            # (membership is read before the update, so cr == ce counts once)
            drop_r = cr >= 0 and cr != ce and sr not in in_topp
            if enter:
                if ev >= 0:
                    del self.topp[ev]
                self.topp.append((a, c, slot))
            if drop_e:
                self.pend.append(se)
            if drop_r:
                self.pend.append(sr)
            if W > 0:
                self.recent[c % W] = slot
            if retained:
                self.slot_cell[slot] = c
            live = {t[2] for t in self.topp} | set(self.recent.values())
            assert len(live) <= W + P
            assert len(live) + len(self.pend) + len(self.free) == self.M
            if c + 1 >= n_row0:
                emit(c + 1)
        self.pos += n_new
        # one row for every candidate count a query of this step has
        assert sorted(rows) == list(range(n_row0, n_end + 1))
        return rows


@pytest.mark.parametrize("W,P,w,max_new,seed", [
    (0, 8, 64, 40, 1), (0, 1, 0, 7, 2), (3, 5, 32, 100, 3), (1, 0, 64, 33, 4),
    (4, 16, 512, 256, 5), (0, 6, 96, 1, 6), (2, 3, 0, 64, 7)])
def test_stream_keep_sets_equal_eq8_over_the_prefix(W, P, w, max_new, seed):
    rng = np.random.default_rng(seed)
    s = 32
    n_tok = 40 * s + w + 17
    n_cells = n_tok // s
    # few distinct values: many ties on a_c, which the newest cell must win
    amax = rng.integers(0, 6, n_cells).astype(np.float64)
    orc = oracle.Oracle()
    p = oracle.make_problem(budget=P, n_recent=W, window=w, cell=s)
    model = StreamModel(W, P, s, w, max_new)
    pos = 0
    while pos < n_tok:
        n_new = int(min(rng.integers(1, max_new + 1), n_tok - pos))
        rows = model.step(amax, n_new)
        for n, entries in rows.items():
            want, _ = orc.prune_row(p, amax, n) if n > 0 else (np.zeros(0, np.int32), 0.0)
            cells = [c for c, _ in entries]
            assert cells == sorted(cells) and cells == list(want), (pos, n)
            for c, sl in entries:       # every slot a row names still holds its cell
                assert model.slot_cell[sl] == c
        pos += n_new


@pytest.mark.parametrize("shape", ["increasing", "decreasing", "constant"])
@pytest.mark.parametrize("W,P", [(1, 1), (2, 2), (0, 3), (3, 0)])
def test_stream_keep_sets_on_monotone_norms(shape, W, P):
    """Rising norms make the cell leaving Recent_W the one TopP evicts (released
    once); falling norms keep the oldest cells; equal norms exercise the tie."""
    s, w, max_new = 32, 64, 50
    n_cells = 60
    base = np.arange(n_cells, dtype=np.float64)
    amax = {"increasing": base, "decreasing": base[::-1].copy(),
            "constant": np.ones(n_cells)}[shape]
    orc = oracle.Oracle()
    p = oracle.make_problem(budget=P, n_recent=W, window=w, cell=s)
    model = StreamModel(W, P, s, w, max_new)
    rng = np.random.default_rng(5)
    n_tok = n_cells * s + w
    while model.pos < n_tok:
        n_new = int(min(rng.integers(1, max_new + 1), n_tok - model.pos))
        for n, entries in model.step(amax, n_new).items():
            want, _ = orc.prune_row(p, amax, n) if n > 0 else (np.zeros(0, np.int32), 0.0)
            assert [c for c, _ in entries] == list(want)
            for c, sl in entries:
                assert model.slot_cell[sl] == c


def test_state_bound_is_independent_of_length():
    """Slots never exceed W + P + ceil(B / s) + 2 however many cells stream past."""
    rng = np.random.default_rng(11)
    W, P, s, w, max_new = 2, 12, 32, 64, 48
    amax = rng.random(5000)
    model = StreamModel(W, P, s, w, max_new)
    pos = 0
    while n_cand(pos, w, s) < 4990:
        model.step(amax, int(rng.integers(1, max_new + 1)))
        pos = model.pos
    assert model.M == W + P + (max_new + s - 1) // s + 2
