"""Benchmark of the FS-L forward (five C-ABI calls) on one MI355X.

A step is one pass of the whole path over one batch of synthetic input, with
the inputs resident in HBM: cell summaries, prefix pruning, scoring + top-K,
window attention, and the sparse readout with the combine (eq. 2) in its
epilogue.  The headline workload is the 64k
prefill (B1 H8 N65536 d128 bf16, K32, P256); the 16k prefill and the 256k
decode are reported alongside.  Per-kernel times come from HIP events recorded
on the launch stream between the calls of the timed steps.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from long_context_fs_amd import synth  # noqa: E402

# MI355X published peaks: HBM3E, dense bf16 MFMA, fp32 (vector and MFMA), fp64 vector.
PEAK = {"hbm_GBs": 8000.0, "mfma_bf16_TFs": 2500.0, "valu_f32_TFs": 157.3, "mfma_f32_TFs": 157.3,
        "valu_f64_TFs": 78.6}
# Threads of the oracle's CPU baseline: the host cores a one-GPU job is allotted
# (16 per GPU), even where the machine shows more.
CPU_SHARE = 16
METRIC = "FreeSolo forward queries/s and TFLOP/s at N=16k/64k/256k; % of MI355X roofline"
PRIMARY = "prefill_b1h8_n65536_d128_bf16"
ALSO = ["prefill_b1h1_n2048_d64_f32", "prefill_b2h16_n4096_d64_bf16",
        "prefill_b1h16_n16384_d64_bf16", "decode_b1h8_n262144_q256_d128_bf16",
        "prefill_b1h8_n65536_d128_bf16_prior"]
# Timed phases of a step; "sparse" is the readout with eq. 2 in its epilogue
# (fs_sparse_attn_combine), so the step has no separate combine pass.
PHASES = ["summaries", "prune", "select", "window", "sparse"]
# Source file of each phase's kernel (for matching stored HBM traffic counters).
PHASE_SRC = {"summaries": "summaries.hip", "prune": "prune.hip", "select": "select.hip",
             "window": "window.hip", "sparse": "sparse.hip", "combine": "combine.hip",
             "rerank": "select.hip", "fsb_beam": "fsb.hip"}
# Engine each phase's kernel uses, which fixes the roofline it is priced against
# (selection issues three bf16 products per algorithmic MAC, priced on the
# algorithmic count; fp32 storage prices the matrix phases at the fp32 peak).
PHASE_ENGINE = {"summaries": "hbm", "prune": "int", "select": "mfma", "window": "mfma",
                "sparse": "mfma", "combine": "hbm", "rerank": "mfma"}


def mfma_peak(wl):
    """Peak (TFLOP/s) the matrix phases of a workload are priced against."""
    return PEAK["mfma_bf16_TFs"] if wl.dtype == "bf16" else PEAK["mfma_f32_TFs"]


def n_cand(wl, i):
    return 0 if i < wl.window else min((i - wl.window) // wl.cell, wl.n_cells)


def algorithmic_work(wl, keep_count=None, n_lo=0):
    """Algorithmic FLOP / bytes per launch of each phase (matmul FLOP = 2 per MAC)."""
    d, s, e = wl.head_dim, wl.cell, (2 if wl.dtype == "bf16" else 4)
    BH = wl.batch * wl.heads
    i = np.arange(wl.q_pos0, wl.q_pos0 + wl.n_q)
    n_i = np.where(i < wl.window, 0, np.minimum((i - wl.window) // wl.cell, wl.n_cells))
    if wl.budget < 0:
        a_i = n_i.astype(np.float64) * BH
    elif keep_count is not None:
        kc = keep_count.reshape(BH, -1)
        a_i = np.zeros(len(i))
        pos = n_i > 0
        a_i[pos] = kc[:, n_i[pos] - n_lo].sum(0)
    else:
        a_i = np.minimum(n_i, wl.budget + wl.n_recent).astype(np.float64) * BH
    win_keys = np.minimum(i, wl.window) + 1
    sel_cells = np.minimum(a_i / BH, wl.topk)
    return {
        "summaries": {"bytes": BH * wl.n_cells * (s * d * e + (d + 1) * 4)},
        "select": {"flop": float(2 * d * a_i.sum())},
        # eq. 12 reranking (not part of the step): every token of every candidate cell
        "rerank": {"flop": float(2 * d * s * a_i.sum())},
        "window": {"flop": float(4 * d * win_keys.sum() * BH)},
        "sparse": {"flop": float(4 * d * s * sel_cells.sum() * BH)},
        "combine": {"bytes": 3 * BH * wl.n_q * d * e},
    }


def step_flop(work):
    """Algorithmic FLOP of one timed step: the matrix phases the step runs (eq. 12
    reranking is timed on its own and is not part of it)."""
    return sum(work[ph].get("flop", 0.0) for ph in PHASES if ph in work)


def kernel_source_sha(phase):
    """Hash of a phase's kernel source and the device headers it includes."""
    h = hashlib.sha256()
    for name in (PHASE_SRC[phase], "mfma_tile.hpp", "fs_device.hpp"):
        h.update(open(os.path.join(ROOT, "long_context_fs_amd", "csrc", name), "rb").read())
    return h.hexdigest()[:16]


def stored_traffic(phase):
    """HBM bytes per launch from committed rocprofv3 counter runs, if the kernel
    source is unchanged since they were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    data = json.load(open(path))
    ent = data.get(phase)
    if not ent:
        return None
    if ent.get("src_sha") != kernel_source_sha(phase):
        return None
    return ent.get("bytes_per_launch")


def run_workload(name, steps, warmup, torch, fs, rerank=False):
    wl = synth.WORKLOADS[name]
    x = synth.generate(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(tdt) for n in ("q", "k", "v"))
    alpha = torch.from_numpy(x["alpha"]).to(dev)
    del x
    fwd = fs.FsForward.for_workload(wl, device=dev)
    p = fwd.prob
    # the window's RoPE table depends only on (w, d, rope_base): built once, like a weight
    fs.fs_window_table(p, fwd.rope_base, fwd.ws)

    def step(ev=None):
        def mark(j):
            if ev is not None:
                ev[j].record()
        mark(0)
        fs.fs_cell_summaries(p, k, fwd.kbar, fwd.amax)
        mark(1)
        if fwd.pruned:
            fs.fs_prune_prefix(p, fwd.amax, fwd.n_recent, fwd.budget, fwd.keep, fwd.keep_count,
                               workspace=fwd.ws_prune)
        mark(2)
        fs.fs_select_topk(p, q, fwd.kbar, fwd.keep, fwd.keep_count, fwd.keep_w, fwd.topk,
                          fwd.idx, None, None, fwd.prior, fwd.ws_select)
        mark(3)
        fs.fs_window_attn_tabled(p, q, k, v, fwd.ws, fwd.o_sr)
        mark(4)
        fs.fs_sparse_attn_combine(p, q, k, v, fwd.idx, fwd.topk, fwd.rms_eps, fwd.o_sr, alpha,
                                  fwd.o, fwd.ws_sparse)
        mark(5)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # whole-step time, no events between the calls
    t0 = time.perf_counter()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / steps
    # per-phase times: events on the launch stream between the calls
    phase_ms = {ph: [] for ph in PHASES}
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(PHASES) + 1)]
        step(ev)
        torch.cuda.synchronize()
        for j, ph in enumerate(PHASES):
            phase_ms[ph].append(ev[j].elapsed_time(ev[j + 1]))
    phase_avg = {ph: float(np.mean(v)) for ph, v in phase_ms.items()}
    phase_pct = {ph: [float(np.percentile(v, q)) for q in (10, 50, 90)]
                 for ph, v in phase_ms.items()}
    # the same step captured once in a HIP graph and replayed (no launch gaps)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(warmup):
        graph.replay()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record()
    for _ in range(steps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / steps
    del graph
    cold_ms = None
    if wl.q_pos0 > 0:
        # decode: every step after a 512 MiB write that evicts L2 and the Infinity Cache
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        cold = []
        for _ in range(steps):
            flush.fill_(1)
            c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            c0.record()
            step()
            c1.record()
            torch.cuda.synchronize()
            cold.append(c0.elapsed_time(c1))
        cold_ms = [float(np.percentile(cold, q)) for q in (10, 50, 90)]
        del flush
    rerank_ms = None
    if rerank:
        # eq. 12 token-level reranking in place of eq. 7's scoring, timed on its own
        rr_idx = torch.empty_like(fwd.idx)
        rr_ws = torch.empty(fs.fs_rerank_workspace_size(p, fwd.keep_w if fwd.pruned else 0),
                            dtype=torch.uint8, device=q.device)

        def rr():
            fs.fs_rerank_topk(p, q, k, fwd.keep, fwd.keep_count, fwd.keep_w, fwd.topk, rr_idx,
                              None, None, fwd.prior, rr_ws)
        for _ in range(warmup):
            rr()
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(steps):
            rr()
        s1.record()
        torch.cuda.synchronize()
        rerank_ms = s0.elapsed_time(s1) / steps
    kc = fwd.keep_count.cpu().numpy() if fwd.pruned else None
    work = algorithmic_work(wl, kc, fwd.n_lo)
    queries = wl.batch * wl.n_q
    total_flop = step_flop(work)
    if rerank_ms is not None:
        phase_avg = dict(phase_avg, rerank=rerank_ms)
    return dict(wl=wl, ms_step=ms_step, wall=wall, phase_ms=phase_avg, work=work,
                qps=queries / (ms_step * 1e-3), tflops=total_flop / (ms_step * 1e-3) / 1e12,
                total_gflop=total_flop / 1e9, phase_pct=phase_pct, cold_ms=cold_ms,
                graph_ms=graph_ms,
                qhps=queries * wl.heads / (ms_step * 1e-3))


def phase_fracs(res):
    """Each timed phase's algorithmic work over its roofline time, divided by the
    measured time (pruning is integer work: time only)."""
    out = {}
    for ph, ms in res["phase_ms"].items():
        eng, w = PHASE_ENGINE.get(ph), res["work"].get(ph, {})
        if eng == "hbm":
            t_roof = w["bytes"] / (PEAK["hbm_GBs"] * 1e9)
        elif eng == "mfma" and "flop" in w:
            t_roof = w["flop"] / (mfma_peak(res["wl"]) * 1e12)
        else:
            continue
        out[ph] = t_roof / (ms * 1e-3)
    return out


def run_stream(torch, fs, decode_steps=200, lengths=(16384, 262144)):
    """Streaming FS-L at the 256k decode shape (B1 H8 d128 bf16, w 512, P 512, K 32):
    a chunked prefill in 256-token steps through the bounded state, then single-token
    decode steps at each context length in `lengths`.  Inputs are N(0, 1) drawn on the
    device with a fixed seed."""
    wl = synth.WORKLOADS["decode_b1h8_n262144_q256_d128_bf16"]
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(12)
    B, H, d, chunk = wl.batch, wl.heads, wl.head_dim, 256
    alpha = torch.rand(H, generator=gen, device=dev)
    out = {"workload": wl.name, "budget": wl.budget, "topk": wl.topk, "window": wl.window,
           "chunk": chunk}

    def rnd(n):
        return torch.randn((B, H, n, d), generator=gen, device=dev).to(torch.bfloat16)

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    for n_ctx in lengths:
        st = fs.FsStream(B, H, d, wl.window, wl.n_recent, wl.budget, wl.topk, chunk,
                         fs.FS_BF16, alpha, rope_base=wl.rope_base, rms_eps=wl.rms_eps,
                         device=dev)
        out["state_bytes"] = st.bytes
        n_ch = n_ctx // chunk
        # the whole context, chunk-major so that every step's tokens are contiguous
        qa, ka, va = (torch.randn((n_ch, B, H, chunk, d), generator=gen, device=dev)
                      .to(torch.bfloat16) for _ in range(3))
        o = torch.empty_like(qa[0])
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for j in range(n_ch):
            st.step(qa[j], ka[j], va[j], o)
        e1.record()
        torch.cuda.synchronize()
        if n_ctx == max(lengths):
            ms = e0.elapsed_time(e1)
            out["prefill_tokens_per_s"] = n_ctx * B / (ms * 1e-3)
            out["prefill_ms_per_chunk"] = ms / (n_ctx // chunk)
        q1, k1, v1 = rnd(1), rnd(1), rnd(1)
        o1 = torch.empty_like(q1)
        for _ in range(10):
            st.step(q1, k1, v1, o1)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record()
        for _ in range(decode_steps):
            st.step(q1, k1, v1, o1)
        e1.record()
        torch.cuda.synchronize()
        out[f"decode_ms_per_token_n{n_ctx}"] = e0.elapsed_time(e1) / decode_steps
        del st, qa, ka, va
    out["decode_tokens_per_s"] = B / (out[f"decode_ms_per_token_n{max(lengths)}"] * 1e-3)
    return out


FSB_BEAM, FSB_SLACK, FSB_TAU_Q = 32, 1.0, 0.7


class FsbSetup:
    """FS-B (section 3.4) at a workload's shape through fs.FsbSelect, with the
    per-head admission thresholds tau_h (the 70% quantile of the head's a_c).
    kbar/amax are the caller's eq. 5 summaries on the device."""

    def __init__(self, torch, fs, wl, p, kbar, amax):
        H, C = wl.heads, wl.n_cells
        self.kbar, self.amax = kbar, amax
        self.tau = torch.quantile(amax[0].reshape(H, C).float(), FSB_TAU_Q, dim=1).contiguous()
        self.sel = fs.FsbSelect(p, wl.topk, FSB_BEAM, FSB_SLACK, device=kbar.device)
        self.idx, self.effort = self.sel.idx, self.sel.effort

    def build(self):
        self.sel.build(self.kbar, self.amax, self.tau)

    def search(self, q, effort=False, k=None):
        self.sel.select(q, effort=effort, k=k)


def run_fsb(name, steps, warmup, torch, fs):
    """FS-B forward at a workload's shape: summaries, both forests, beam search of
    width FSB_BEAM (slack FSB_SLACK), then the FS-L window and the readout with eq. 2 in
    its epilogue."""
    wl = synth.WORKLOADS[name]
    x = synth.generate(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(tdt) for n in ("q", "k", "v"))
    alpha = torch.from_numpy(x["alpha"]).to(dev)
    del x
    fwd = fs.FsForward.for_workload(wl, device=dev)
    p = fwd.prob
    fs.fs_cell_summaries(p, k, fwd.kbar, fwd.amax)
    fs.fs_window_table(p, fwd.rope_base, fwd.ws)
    fb = FsbSetup(torch, fs, wl, p, fwd.kbar, fwd.amax)
    calls = [("summaries", lambda: fs.fs_cell_summaries(p, k, fwd.kbar, fwd.amax)),
             ("forest_build", fb.build),
             ("beam_select", lambda: fb.search(q)),
             ("window", lambda: fs.fs_window_attn_tabled(p, q, k, v, fwd.ws, fwd.o_sr)),
             ("sparse", lambda: fs.fs_sparse_attn_combine(p, q, k, v, fb.idx, wl.topk,
                                                          fwd.rms_eps, fwd.o_sr, alpha, fwd.o,
                                                          fwd.ws_sparse))]

    def step(ev=None):
        for j, (_, fn) in enumerate(calls):
            if ev is not None:
                ev[j].record()
            fn()
        if ev is not None:
            ev[-1].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    times = {nm: [] for nm, _ in calls}
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
        step(ev)
        torch.cuda.synchronize()
        for j, (nm, _) in enumerate(calls):
            times[nm].append(ev[j].elapsed_time(ev[j + 1]))
    phase_ms = {nm: float(np.mean(t)) for nm, t in times.items()}
    # the same search with eq. 12's token-level reranking of the found cells
    rr = []
    for _ in range(steps):
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record()
        fb.search(q, k=k)
        ev[1].record()
        torch.cuda.synchronize()
        rr.append(ev[0].elapsed_time(ev[1]))
    fb.search(q, effort=True)
    torch.cuda.synchronize()
    scored = int(fb.effort.to(torch.int64).sum().item())
    nq = wl.batch * wl.heads * wl.n_q
    # algorithmic work of one search launch: a d-long fp64 dot product (2d flops)
    # per scored node; the node rows it reads (mean row + rho, A, first cell) come
    # from a forest of a few tens of MB held in the caches, so HBM does not bound it
    e = 2 if wl.dtype == "bf16" else 4
    flop_beam = scored * 2.0 * wl.head_dim
    bytes_beam = scored * (4 * wl.head_dim + 12) + nq * (wl.head_dim * e + 4 * wl.topk)
    t = phase_ms["beam_select"] * 1e-3
    ach = flop_beam / t / 1e12
    return {"workload": wl.name, "beam": FSB_BEAM, "slack": FSB_SLACK,
            "tau": f"per head, the {FSB_TAU_Q:.0%} quantile of its a_c",
            "ms_per_step": ms_step, "queries_per_s": wl.batch * wl.n_q / (ms_step * 1e-3),
            "phase_ms": phase_ms, "beam_select_rerank_ms": float(np.mean(rr)),
            "nodes_scored_per_query_head": scored / nq,
            "roofline": {"bound": "alu", "achieved": ach, "peak": PEAK["valu_f64_TFs"],
                         "unit": "TFLOP/s", "frac": ach / PEAK["valu_f64_TFs"],
                         "traffic": stored_traffic("fsb_beam") if name == PRIMARY else None,
                         "kernel": "beam_select", "flop_per_launch": flop_beam,
                         "node_bytes_per_launch": bytes_beam,
                         "node_bytes_GBs": bytes_beam / t / 1e9,
                         "ms_per_launch": phase_ms["beam_select"]}}


def roofline(res, ph=None):
    """Roofline entry for phase `ph`, by default the one that takes the most time."""
    if ph is None:
        ph = max((p for p in PHASES if p != "prune"), key=lambda p: res["phase_ms"][p])
    t = res["phase_ms"][ph] * 1e-3
    eng = PHASE_ENGINE[ph]
    w = res["work"][ph]
    traffic = stored_traffic(ph) if res["wl"].name == PRIMARY else None
    if eng == "hbm":
        ach = w["bytes"] / t / 1e9
        out = {"bound": "hbm", "achieved": ach, "peak": PEAK["hbm_GBs"], "unit": "GB/s"}
    else:
        ach = w["flop"] / t / 1e12
        out = {"bound": "mfma", "achieved": ach, "peak": mfma_peak(res["wl"]), "unit": "TFLOP/s"}
    out["frac"] = out["achieved"] / out["peak"]
    out["traffic"] = traffic
    out["kernel"] = ph
    out["ms_per_launch"] = res["phase_ms"][ph]
    return out


def cpu_baseline(name, budget_s=15.0):
    """The fp64 oracle on a bounded sample of query rows of the workload: random
    rows of head 0, and of further heads when one head's rows take less than the
    budget."""
    import oracle
    wl = synth.WORKLOADS[name]
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, CPU_SHARE))
    p = oracle.problem_from(wl.replace(batch=1, heads=1))
    orc = oracle.Oracle()
    rng = np.random.default_rng(0)

    def head_data(x, hh):
        t0 = time.perf_counter()
        kbar, amax = orc.cell_summaries_head(p, x["k"][0, hh])
        return kbar, amax, time.perf_counter() - t0

    x = synth.generate(wl.replace(batch=1, heads=1))
    kbar, amax, t_sum = head_data(x, 0)
    n_try = min(64, wl.n_q)
    rows = np.sort(rng.choice(wl.n_q, n_try, replace=False))
    t0 = time.perf_counter()
    orc.forward_rows(p, x["q"][0, 0], x["k"][0, 0], x["v"][0, 0], kbar, amax, 1.0, rows,
                     nthreads=cores)
    t_try = time.perf_counter() - t0
    want = int(max(n_try, n_try * budget_s / max(t_try, 1e-3)))
    n_heads = int(min(wl.heads, max(1, -(-want // wl.n_q))))
    if n_heads > 1:
        x = synth.generate(wl.replace(batch=1, heads=n_heads))
    n_rows, t_rows, t_sums = 0, 0.0, 0.0
    for hh in range(n_heads):
        if hh > 0 or n_heads > 1:
            kbar, amax, t_sum = head_data(x, hh)
        t_sums += t_sum
        take = int(min(wl.n_q, want - n_rows))
        rows = np.sort(rng.choice(wl.n_q, take, replace=False))
        t0 = time.perf_counter()
        orc.forward_rows(p, x["q"][0, hh], x["k"][0, hh], x["v"][0, hh], kbar, amax, 1.0, rows,
                         nthreads=cores)
        t_rows += time.perf_counter() - t0
        n_rows += take
    # per-query cost, with each head's summaries spread over all of its queries
    per_q = t_rows / n_rows + t_sums / n_heads / wl.n_q
    cpu = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": 1.0 / per_q, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "cpu": cpu, "cores_note": f"threads = the job's affinity cores, at most the "
                                      f"{CPU_SHARE} host cores allotted per GPU",
            "sample": f"{n_rows} random query rows of {n_heads} head(s) of {name} "
                      f"({t_rows:.1f} s on {cores} threads) + those heads' cell summaries "
                      f"({t_sums:.2f} s, amortised over {wl.n_q} queries per head)"}


# ---- profiling helpers (rocprofv3 drives these; the summaries go to profiles/) ----
def run_phase(name, phase, reps, torch, fs):
    """One full forward, then `reps` launches of a single phase (counter runs)."""
    wl = synth.get_workload(name)
    x = synth.generate(wl)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x[n]).to(dev).to(tdt) for n in ("q", "k", "v"))
    alpha = torch.from_numpy(x["alpha"]).to(dev)
    f = fs.FsForward.for_workload(wl, device=dev)
    f(q, k, v, alpha)
    p = f.prob
    rr_ws = torch.empty(fs.fs_rerank_workspace_size(p, f.keep_w if f.pruned else 0),
                        dtype=torch.uint8, device=dev)
    fb = FsbSetup(torch, fs, wl, p, f.kbar, f.amax) if phase.startswith("fsb_") else None
    if fb is not None:
        fb.build()
    calls = {
        "fsb_forest": lambda: fb.build(),
        "fsb_beam": lambda: fb.search(q),
        "fsb_all": lambda: (fb.build(), fb.search(q)),
        "summaries": lambda: fs.fs_cell_summaries(p, k, f.kbar, f.amax),
        "prune": lambda: fs.fs_prune_prefix(p, f.amax, f.n_recent, f.budget, f.keep,
                                            f.keep_count, workspace=f.ws_prune),
        "select": lambda: fs.fs_select_topk(p, q, f.kbar, f.keep, f.keep_count, f.keep_w,
                                            f.topk, f.idx, None, None, f.prior, f.ws_select),
        "rerank": lambda: fs.fs_rerank_topk(p, q, k, f.keep, f.keep_count, f.keep_w, f.topk,
                                            f.idx, None, None, f.prior, rr_ws),
        "window": lambda: fs.fs_window_attn_tabled(p, q, k, v, f.ws, f.o_sr),
        "sparse": lambda: fs.fs_sparse_attn_combine(p, q, k, v, f.idx, f.topk, f.rms_eps, f.o_sr,
                                                    alpha, f.o, f.ws_sparse),
        "combine": lambda: fs.fs_combine(p, f.o_sr, f.o_lr, alpha, f.o),
    }
    for _ in range(reps):
        calls[phase]()
    torch.cuda.synchronize()
    print(f"phase {phase} of {wl.name}: {reps} launches", flush=True)


def run_copy(mib, reps, torch):
    """A plain device copy of a known size: calibrates the HBM byte counters."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copy {mib} MiB x {reps}", flush=True)


def _rocpd_rows(db, query):
    import sqlite3
    con = sqlite3.connect(db)
    try:
        return list(con.execute(query))
    finally:
        con.close()


def kernel_stats(db):
    """[(name, calls, average us, total us)] from a --kernel-trace run."""
    return [(r[0], int(r[1]), float(r[3]), float(r[2])) for r in _rocpd_rows(
        db, "select name, total_calls, total_duration, average from top_kernels")]


def counter_means(db, substr):
    """{counter: mean over dispatches of the kernel (summed over hardware units)}."""
    per = {}
    for disp, kname, cname, val in _rocpd_rows(
            db, "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        if substr in kname:
            per.setdefault(disp, {}).setdefault(cname, 0.0)
            per[disp][cname] += val
    if not per:
        return {}
    names = set().union(*per.values())
    return {c: sum(d.get(c, 0.0) for d in per.values()) / len(per) for c in names}


def write_traffic(phase, kernel_substr, fetch_db, write_db, copy_fetch_db, copy_write_db,
                  copy_mib):
    """Record HBM bytes per launch of one phase's kernel in profiles/traffic.json."""
    write_traffic_kib(phase, kernel_substr,
                      counter_means(fetch_db, kernel_substr)["FETCH_SIZE"],
                      counter_means(write_db, kernel_substr)["WRITE_SIZE"],
                      counter_means(copy_fetch_db, "copy")["FETCH_SIZE"],
                      counter_means(copy_write_db, "copy")["WRITE_SIZE"], copy_mib)


def write_traffic_jsonl(phase, kernel_substr, path_jsonl, copy_mib):
    """Same, from per-dispatch counter means already reduced to JSON lines
    ({"tag": counter, "kernel": substring, "counters": {...}})."""
    kib = {}
    for line in open(path_jsonl):
        r = json.loads(line)
        kib[(r["kernel"], r["tag"])] = r["counters"][r["tag"]]
    write_traffic_kib(phase, kernel_substr, kib[(kernel_substr, "FETCH_SIZE")],
                      kib[(kernel_substr, "WRITE_SIZE")], kib[("copy", "FETCH_SIZE")],
                      kib[("copy", "WRITE_SIZE")], copy_mib)


def write_traffic_kib(phase, kernel_substr, fetch_kib, write_kib, copy_fetch_kib,
                      copy_write_kib, copy_mib):
    copy_bytes = copy_mib * (1 << 20)
    f_copy = copy_fetch_kib * 1024 / copy_bytes
    w_copy = copy_write_kib * 1024 / copy_bytes
    fetch = fetch_kib * 1024 / f_copy
    write = write_kib * 1024 / w_copy
    path = os.path.join(ROOT, "profiles", "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    data[phase] = {"kernel": kernel_substr, "src_sha": kernel_source_sha(phase),
        "fetch_bytes_per_launch": fetch,
        "write_bytes_per_launch": write, "bytes_per_launch": fetch + write,
        "copy_factor_fetch": f_copy, "copy_factor_write": w_copy, "copy_mib": copy_mib}
    json.dump(data, open(path, "w"), indent=1, sort_keys=True)
    print(json.dumps(data[phase]))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only-primary", action="store_true")
    ap.add_argument("--phase", help="profiling: launch only this phase --reps times")
    ap.add_argument("--workload", default=PRIMARY, help="workload of --phase")
    ap.add_argument("--reps", type=int, default=3)
    ap.add_argument("--copy-mib", type=int, help="profiling: plain copy of this many MiB")
    ap.add_argument("--kernel-stats", metavar="DB", help="print kernel stats of a rocpd db")
    ap.add_argument("--write-traffic", nargs=6, metavar=("PHASE", "KERNEL", "FETCH_DB",
                    "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"))
    ap.add_argument("--write-traffic-jsonl", nargs=3, metavar=("PHASE", "KERNEL", "JSONL"))
    args = ap.parse_args()
    if args.kernel_stats:
        for name, calls, avg, tot in kernel_stats(args.kernel_stats):
            print(f"{avg:12.2f} us avg  {calls:5d} calls  {tot / 1e3:10.3f} ms total  {name[:110]}")
        return
    if args.write_traffic:
        write_traffic(*args.write_traffic, copy_mib=args.copy_mib or 1024)
        return
    if args.write_traffic_jsonl:
        write_traffic_jsonl(*args.write_traffic_jsonl, copy_mib=args.copy_mib or 1024)
        return
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported. "
              "Heads and batch shard across GPUs with no communication; that path is not implemented.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from long_context_fs_amd import fs
    fs.load()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_mib and not args.phase:
        run_copy(args.copy_mib, args.reps, torch)
        return
    if args.phase == "stream":
        print(json.dumps(run_stream(torch, fs, decode_steps=args.reps, lengths=(262144,))),
              flush=True)
        return
    if args.phase:
        run_phase(args.workload, args.phase, args.reps, torch, fs)
        return

    main_res = run_workload(PRIMARY, args.steps, args.warmup, torch, fs, rerank=True)
    also = {}
    if not args.only_primary:
        for name in ALSO:
            r = run_workload(name, args.steps, args.warmup, torch, fs)
            also[name] = {"queries_per_s": r["qps"], "query_heads_per_s": r["qhps"],
                          "ms_per_step": r["ms_step"], "graph_ms_per_step": r["graph_ms"],
                          "tflops": r["tflops"], "gflop_per_step": r["total_gflop"],
                          "phase_ms": r["phase_ms"], "phase_ms_p10_p50_p90": r["phase_pct"],
                          "phase_roofline_frac": phase_fracs(r), "roofline": roofline(r)}
            if r["cold_ms"] is not None:
                also[name]["cold_ms_per_step_p10_p50_p90"] = r["cold_ms"]
    stream = None if args.only_primary else run_stream(torch, fs)
    fsb = None if args.only_primary else run_fsb(PRIMARY, max(2, args.steps // 4), 2, torch, fs)
    wl = main_res["wl"]
    out = {
        "metric": METRIC,
        "value": main_res["qps"],
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_step"],
        "graph_ms_per_step": main_res["graph_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v with a planted needle cell)",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads,
                   "seq_len": wl.n_ctx, "n_q": wl.n_q, "head_dim": wl.head_dim,
                   "window": wl.window, "cell": wl.cell, "topk": wl.topk, "budget": wl.budget},
        "tflops": main_res["tflops"],
        "gflop_per_step": main_res["total_gflop"],
        "phase_ms": main_res["phase_ms"],
        "phase_ms_p10_p50_p90": main_res["phase_pct"],
        "phase_roofline_frac": phase_fracs(main_res),
        "query_heads_per_s": main_res["qhps"],
        "roofline": roofline(main_res),
        "rerank": roofline(main_res, "rerank"),
        "also": also,
        "stream": stream,
        "fsb": fsb,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(PRIMARY)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
