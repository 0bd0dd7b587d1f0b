"""Helpers for the GPU-vs-oracle parity tests (test code only)."""
from __future__ import annotations

import numpy as np

TIE_REL = 1e-5           # near-tie threshold for the top-K and top-P boundaries
TOL = {"f32": 1e-4, "bf16": 2e-2}


def to_dev(x: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    return t.to(torch.bfloat16) if dtype == "bf16" else t.to(torch.float32)


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> np.ndarray:
    """Per row: max |got - ref| / max |ref| (absolute error where the row is 0)."""
    got = got.reshape(-1, got.shape[-1]).astype(np.float64)
    ref = ref.reshape(-1, ref.shape[-1]).astype(np.float64)
    den = np.abs(ref).max(-1)
    num = np.abs(got - ref).max(-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def topk_boundary(scores: np.ndarray, cells: np.ndarray, k: int):
    """(K-th, (K+1)-th) largest scores under the (score, cell) descending order."""
    order = np.lexsort((-cells, -scores))
    s = scores[order]
    return (s[k - 1] if len(s) >= k else None, s[k] if len(s) > k else None)


def accept_set(gpu: np.ndarray, cand: np.ndarray, scores: np.ndarray, k: int,
               want: np.ndarray) -> str:
    """Check a set chosen by the GPU against the oracle's scores of the candidates.

    'exact' when it equals the oracle's set; 'tie' when they differ only across
    a boundary whose relative gap is below TIE_REL (every chosen cell then
    scores at least r_K - TIE_REL * max(|r_K|, |r_K+1|)); raises otherwise."""
    gpu = np.sort(np.asarray(gpu))
    want = np.sort(np.asarray(want))
    assert len(gpu) == min(k, len(cand)), (len(gpu), k, len(cand))
    assert len(np.unique(gpu)) == len(gpu) and np.isin(gpu, cand).all()
    if np.array_equal(gpu, want):
        return "exact"
    rk, rk1 = topk_boundary(scores, cand, k)
    assert rk is not None and rk1 is not None
    scale = max(abs(rk), abs(rk1))
    gap = (rk - rk1) / scale if scale > 0 else 0.0
    assert gap < TIE_REL, f"selection differs away from a near-tie (gap {gap:.3g})"
    got_scores = scores[np.searchsorted(cand, gpu)] if np.all(np.diff(cand) > 0) else \
        np.array([scores[np.where(cand == c)[0][0]] for c in gpu])
    assert got_scores.min() >= rk - TIE_REL * scale, "GPU chose a cell below the near-tie band"
    return "tie"
