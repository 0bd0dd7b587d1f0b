"""Seeded synthetic inputs for the FreeSolo FS-L attention forward.

This module is the only code shared by the HIP path and the CPU oracle.  It
draws inputs and holds none of the method's arithmetic: no RoPE, no cell
summaries, no pruning, no scoring, no attention.

The workloads stand in for the long-context retrieval settings of the FreeSolo
paper summary (picx.dev page, "Key Findings": single needles at 256k; "Empirical
Scaling": 4k to 256k contexts).  They are synthetic: i.i.d. N(0,1) queries,
keys and values, plus the planted structure each workload names (per-head key
scales, a few high-norm cells, or one "needle" cell aligned with the last
queries).  No benchmark items are reproduced.

Draw order, from ``numpy.random.Generator(PCG64(seed))``:
  1. q  [B, H, n_q, d]   standard normal, float32
  2. k  [B, H, N, d]     standard normal, float32
  3. v  [B, H, N, d]     standard normal, float32
  4. the structure (per-head key scales / hot cells / needles, in (b, h) order)
  5. alpha [H]           (only when drawn, U[0, 1])
Then every tensor is rounded to the storage dtype: bf16 by round-to-nearest-
even from the float32 draw.  Arrays are returned as float32 holding exactly
the stored values, so both sides read identical numbers.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field

import numpy as np

__all__ = ["Workload", "WORKLOADS", "get_workload", "generate", "round_bf16", "bf16_bits"]


@dataclass(frozen=True)
class Workload:
    """Shape, hyper-parameters and planted structure of one forward problem."""

    name: str
    batch: int
    heads: int
    n_ctx: int            # N: keys/values at positions 0..N-1
    head_dim: int         # d
    dtype: str            # "f32" or "bf16" (storage dtype of q, k, v and outputs)
    n_q: int              # queries at positions q_pos0 .. q_pos0+n_q-1
    q_pos0: int
    topk: int             # K cells per query
    budget: int           # P cells kept by max-norm priority; < 0 means no pruning
    n_recent: int = 0     # W most recent candidate cells always kept
    cell: int = 32        # s
    window: int = 512     # w (look-back radius)
    rope_base: float = 10000.0
    rms_eps: float = 1e-6
    structure: str = "iid"          # iid | key_scale | hot_cells | needle
    hot_frac: float = 0.0           # fraction of cells given 3x keys (hot_cells)
    needle_queries: int = 0         # last queries aligned with the needle
    alpha: float | None = None      # fixed alpha for every head; None = U[0,1] per head
    seed: int = 0
    prior_lambda: float = 0.0       # eq. 7 prior: head h uses lambda * (h + 1) / H ...
    prior_sigma: float = 0.0        # ... and sigma * 2^(h mod 4); lambda 0 = no prior

    @property
    def n_cells(self) -> int:
        return self.n_ctx // self.cell

    def prior_arrays(self):
        """Per-head (lambda_h, sigma_h) as float32 arrays, or (None, None)."""
        if self.prior_lambda <= 0:
            return None, None
        h = np.arange(self.heads)
        lam = np.float32(self.prior_lambda) * (h + 1).astype(np.float32) / np.float32(self.heads)
        sig = np.float32(self.prior_sigma) * np.float32(2.0) ** (h % 4).astype(np.float32)
        return lam.astype(np.float32), sig.astype(np.float32)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: shapes, dtypes and structure of the FS-L settings.
WORKLOADS = {
    "prefill_b1h1_n2048_d64_f32": Workload(
        name="prefill_b1h1_n2048_d64_f32", batch=1, heads=1, n_ctx=2048, head_dim=64,
        dtype="f32", n_q=2048, q_pos0=0, topk=8, budget=-1, alpha=0.5, seed=1),
    "prefill_b2h16_n4096_d64_bf16": Workload(
        name="prefill_b2h16_n4096_d64_bf16", batch=2, heads=16, n_ctx=4096, head_dim=64,
        dtype="bf16", n_q=4096, q_pos0=0, topk=16, budget=64, structure="key_scale", seed=2),
    "prefill_b1h16_n16384_d64_bf16": Workload(
        name="prefill_b1h16_n16384_d64_bf16", batch=1, heads=16, n_ctx=16384, head_dim=64,
        dtype="bf16", n_q=16384, q_pos0=0, topk=16, budget=128, structure="hot_cells",
        hot_frac=0.01, seed=3),
    "prefill_b1h8_n65536_d128_bf16": Workload(
        name="prefill_b1h8_n65536_d128_bf16", batch=1, heads=8, n_ctx=65536, head_dim=128,
        dtype="bf16", n_q=65536, q_pos0=0, topk=32, budget=256, structure="needle",
        needle_queries=64, seed=4),
    "decode_b1h8_n262144_q256_d128_bf16": Workload(
        name="decode_b1h8_n262144_q256_d128_bf16", batch=1, heads=8, n_ctx=262144,
        head_dim=128, dtype="bf16", n_q=256, q_pos0=262144 - 256, topk=32, budget=512,
        structure="needle", needle_queries=256, seed=5),
    # the 64k prefill with eq. 7's position prior switched on (lambda_h up to 0.1,
    # sigma_h from 2048 to 16384 tokens)
    "prefill_b1h8_n65536_d128_bf16_prior": Workload(
        name="prefill_b1h8_n65536_d128_bf16_prior", batch=1, heads=8, n_ctx=65536,
        head_dim=128, dtype="bf16", n_q=65536, q_pos0=0, topk=32, budget=256,
        structure="needle", needle_queries=64, seed=4, prior_lambda=0.1, prior_sigma=2048.0),
}

# Short aliases in the order the workloads are listed above.
ALIASES = {f"c{i + 1}": name for i, name in enumerate(WORKLOADS)}


def get_workload(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty_like(x)
    flat_in = x.reshape(-1)
    flat_out = out.reshape(-1)
    step = 1 << 24
    for s in range(0, flat_in.size, step):
        u = flat_in[s:s + step].view(np.uint32)
        r = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
        flat_out[s:s + step] = (r & np.uint32(0xFFFF0000)).view(np.float32)
    return out


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> np.uint32(16)).astype(np.uint16)


def _first_candidate_count(pos: int, window: int, cell: int) -> int:
    # Number of complete cells that end before pos - window.  This only places
    # the needle where the aligned queries can reach it (input construction).
    return 0 if pos < window else (pos - window) // cell


def generate(wl: Workload, seed: int | None = None) -> dict:
    """Draw the inputs of ``wl``.  Returns a dict of numpy arrays and metadata."""
    rng = np.random.Generator(np.random.PCG64(wl.seed if seed is None else seed))
    B, H, N, d, s = wl.batch, wl.heads, wl.n_ctx, wl.head_dim, wl.cell
    q = rng.standard_normal((B, H, wl.n_q, d), dtype=np.float32)
    k = rng.standard_normal((B, H, N, d), dtype=np.float32)
    v = rng.standard_normal((B, H, N, d), dtype=np.float32)
    meta: dict = {}

    if wl.structure == "key_scale":
        scale = rng.uniform(0.5, 2.0, size=H).astype(np.float32)
        k *= scale[None, :, None, None]
        meta["key_scale"] = scale
    elif wl.structure == "hot_cells":
        n_hot = int(round(wl.hot_frac * wl.n_cells))
        hot = np.zeros((B, H, n_hot), dtype=np.int64)
        for b in range(B):
            for h in range(H):
                cells = np.sort(rng.choice(wl.n_cells, size=n_hot, replace=False))
                hot[b, h] = cells
                for c in cells:
                    k[b, h, c * s:(c + 1) * s] *= np.float32(3.0)
        meta["hot_cells"] = hot
    elif wl.structure == "needle":
        nq_al = min(wl.needle_queries, wl.n_q)
        first_aligned = wl.q_pos0 + wl.n_q - nq_al
        reach = _first_candidate_count(first_aligned, wl.window, s)
        if reach < 1:
            raise ValueError("needle workload: aligned queries see no complete cell")
        needle = np.zeros((B, H), dtype=np.int64)
        for b in range(B):
            for h in range(H):
                c = int(rng.integers(0, reach))
                needle[b, h] = c
                u = rng.standard_normal(d)
                u /= np.linalg.norm(u)
                blk = k[b, h, c * s:(c + 1) * s].astype(np.float64)
                norms = np.linalg.norm(blk, axis=1, keepdims=True)
                k[b, h, c * s:(c + 1) * s] = (3.0 * norms * u[None, :]).astype(np.float32)
                for t in range(wl.n_q - nq_al, wl.n_q):
                    e = rng.standard_normal(d)
                    e -= (e @ u) * u
                    e /= np.linalg.norm(e)
                    qn = np.linalg.norm(q[b, h, t].astype(np.float64))
                    q[b, h, t] = (qn * (0.9 * u + np.sqrt(0.19) * e)).astype(np.float32)
        meta["needle"] = needle
        meta["needle_first_query"] = wl.n_q - nq_al
    elif wl.structure != "iid":
        raise ValueError(f"unknown structure {wl.structure!r}")

    if wl.alpha is None:
        alpha = rng.uniform(0.0, 1.0, size=H)
    else:
        alpha = np.full(H, wl.alpha)
    alpha = alpha.astype(np.float32)

    if wl.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif wl.dtype != "f32":
        raise ValueError(f"unknown dtype {wl.dtype!r}")
    return {"q": q, "k": k, "v": v, "alpha": alpha, "meta": meta, "workload": wl}
