"""Host-side checks of bench.py's contract (no GPU): the multi-GPU refusal, the
copy-scaled HBM traffic arithmetic, and the algorithmic work of a small workload
against a direct count of its pairs."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from long_context_fs_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU only" in r.stderr


def test_traffic_is_scaled_by_the_copy_reading(tmp_path, monkeypatch):
    """A copy of 1 GiB whose FETCH_SIZE reads half its bytes doubles a kernel's
    FETCH_SIZE; WRITE_SIZE reads true bytes and is kept."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_sha", lambda phase: "sha")
    lines = [{"tag": "FETCH_SIZE", "kernel": "k", "counters": {"FETCH_SIZE": 1000.0}},
             {"tag": "WRITE_SIZE", "kernel": "k", "counters": {"WRITE_SIZE": 300.0}},
             {"tag": "FETCH_SIZE", "kernel": "copy", "counters": {"FETCH_SIZE": 524288.0}},
             {"tag": "WRITE_SIZE", "kernel": "copy", "counters": {"WRITE_SIZE": 1048576.0}}]
    jl = tmp_path / "c.jsonl"
    jl.write_text("\n".join(json.dumps(x) for x in lines) + "\n")
    bench.write_traffic_jsonl("ph", "k", str(jl), 1024)
    ent = json.load(open(prof / "traffic.json"))["ph"]
    assert ent["fetch_bytes_per_launch"] == 2000.0 * 1024
    assert ent["write_bytes_per_launch"] == 300.0 * 1024
    assert ent["bytes_per_launch"] == 2300.0 * 1024
    assert bench.stored_traffic("ph") == 2300.0 * 1024


def test_algorithmic_work_counts_pairs():
    """Window pairs, candidate cells and selected cells of a small unpruned
    workload, counted one query at a time."""
    wl = synth.get_workload("c1").replace(n_ctx=1300, n_q=1300)
    w = bench.algorithmic_work(wl)
    d, s, K = wl.head_dim, wl.cell, wl.topk
    win = sum(min(i, wl.window) + 1 for i in range(wl.n_q))
    cand = sum(bench.n_cand(wl, i) for i in range(wl.n_q))
    sel = sum(min(bench.n_cand(wl, i), K) for i in range(wl.n_q))
    assert w["window"]["flop"] == 4 * d * win
    assert w["select"]["flop"] == 2 * d * cand
    assert w["sparse"]["flop"] == 4 * d * s * sel
    assert w["combine"]["bytes"] == 3 * wl.n_q * d * 4
    assert w["summaries"]["bytes"] == wl.n_cells * (s * d * 4 + (d + 1) * 4)
    assert np.isclose(w["rerank"]["flop"], 2 * d * s * cand)


def test_step_flop_is_the_timed_phases_only():
    """The step's FLOP total is selection + window + readout; eq. 12 reranking is
    timed on its own and stays out of it."""
    wl = synth.get_workload("c4")
    w = bench.algorithmic_work(wl)
    assert bench.step_flop(w) == w["select"]["flop"] + w["window"]["flop"] + w["sparse"]["flop"]
    assert "rerank" not in bench.PHASES


def test_matrix_phases_are_priced_at_their_dtype_peak():
    assert bench.mfma_peak(synth.get_workload("c1")) == 157.3      # fp32 storage
    assert bench.mfma_peak(synth.get_workload("c4")) == 2500.0     # bf16
    assert bench.PEAK["valu_f32_TFs"] == 157.3 and bench.PEAK["valu_f64_TFs"] == 78.6
    assert set(bench.ALSO) >= {"prefill_b1h1_n2048_d64_f32", "prefill_b2h16_n4096_d64_bf16"}
