"""Thin ctypes binding of libfs.so, the C ABI declared in include/fs.h.

Argument marshalling only: every step of the forward runs in the HIP kernels
of libfs.so.  PyTorch supplies device memory (tensor data pointers) and the
current HIP stream.  There is no fallback: if the library is missing, every
call raises FsError.
"""
from __future__ import annotations

import ctypes as C
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfs.so")

FS_F32, FS_BF16 = 0, 1
CELL = 32

SYMBOLS = ("fs_cell_summaries", "fs_prune_rows", "fs_prune_prefix", "fs_prune_workspace_size",
           "fs_select_topk",
           "fs_workspace_size", "fs_window_attn", "fs_window_table", "fs_window_attn_tabled",
           "fs_sparse_workspace_size", "fs_sparse_attn",
           "fs_sparse_attn_noalloc", "fs_sparse_attn_combine", "fs_combine", "fs_rerank_topk", "fs_rerank_workspace_size",
           "fs_select_workspace_size", "fs_stream_state_size", "fs_stream_reset",
           "fs_stream_step", "fs_forest_size", "fs_forest_build", "fs_beam_select",
           "fs_status_string", "fs_last_error", "fs_last_path")


class FsError(RuntimeError):
    """A libfs call returned an error status, or the library is missing."""

    def __init__(self, msg: str, status: int = -1):
        super().__init__(msg)
        self.status = status


class FsProblem(C.Structure):
    _fields_ = [("batch", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("n_ctx", C.c_int32), ("n_q", C.c_int32), ("q_pos0", C.c_int32),
                ("cell", C.c_int32), ("window", C.c_int32), ("dtype", C.c_int32),
                ("reserved", C.c_int32), ("q_stride", C.c_int64 * 3),
                ("kv_stride", C.c_int64 * 3), ("o_stride", C.c_int64 * 3)]


class FsStreamConfig(C.Structure):
    _fields_ = [("batch", C.c_int32), ("heads", C.c_int32), ("head_dim", C.c_int32),
                ("cell", C.c_int32), ("window", C.c_int32), ("n_recent", C.c_int32),
                ("budget", C.c_int32), ("topk", C.c_int32), ("max_new", C.c_int32),
                ("dtype", C.c_int32), ("rope_base", C.c_float), ("rms_eps", C.c_float)]


_lib = None


def load(path: str | None = None):
    """Load libfs.so (once) and declare the signatures of include/fs.h."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or LIB_PATH
    if not os.path.exists(path):
        raise FsError(f"{path} is not built; run __graft_entry__.build() first")
    L = C.CDLL(path)
    P, vp, i32, f32 = C.POINTER(FsProblem), C.c_void_p, C.c_int32, C.c_float
    sig = {
        "fs_cell_summaries": [P, vp, vp, vp, vp],
        "fs_prune_rows": [P, C.POINTER(i32), C.POINTER(i32)],
        "fs_prune_prefix": [P, vp, i32, i32, vp, vp, vp, C.c_size_t, vp],
        "fs_prune_workspace_size": [P, C.POINTER(C.c_size_t)],
        "fs_select_topk": [P, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, C.c_size_t,
                           vp],
        "fs_select_workspace_size": [P, i32, i32, C.POINTER(C.c_size_t)],
        "fs_rerank_topk": [P, vp, vp, vp, vp, vp, vp, vp, i32, i32, vp, vp, vp, C.c_size_t,
                           vp],
        "fs_rerank_workspace_size": [P, i32, C.POINTER(C.c_size_t)],
        "fs_workspace_size": [P, C.POINTER(C.c_size_t)],
        "fs_window_attn": [P, vp, vp, vp, f32, vp, C.c_size_t, vp, vp],
        "fs_window_table": [P, f32, vp, C.c_size_t, vp],
        "fs_window_attn_tabled": [P, vp, vp, vp, vp, C.c_size_t, vp, vp],
        "fs_sparse_workspace_size": [P, C.POINTER(C.c_size_t)],
        "fs_sparse_attn": [P, vp, vp, vp, vp, i32, f32, vp, C.c_size_t, vp, vp],
        "fs_sparse_attn_noalloc": [P, vp, vp, vp, vp, i32, f32, vp, vp],
        "fs_sparse_attn_combine": [P, vp, vp, vp, vp, i32, f32, vp, vp, vp, C.c_size_t, vp, vp],
        "fs_combine": [P, vp, vp, vp, vp, vp],
        "fs_forest_size": [P, C.POINTER(C.c_size_t)],
        "fs_forest_build": [P, vp, vp, vp, vp, vp],
        "fs_beam_select": [P, vp, vp, vp, vp, i32, f32, vp, vp, i32, vp, vp, vp, vp],
        "fs_stream_state_size": [C.POINTER(FsStreamConfig), C.POINTER(C.c_size_t)],
        "fs_stream_reset": [C.POINTER(FsStreamConfig), vp, C.c_size_t, vp],
        "fs_stream_step": [C.POINTER(FsStreamConfig), vp, C.c_size_t, C.c_int64, i32, vp, vp,
                           vp, vp, vp, vp, vp, vp, vp],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = C.c_int
    L.fs_status_string.argtypes = [C.c_int]
    L.fs_status_string.restype = C.c_char_p
    L.fs_last_error.argtypes = []
    L.fs_last_error.restype = C.c_char_p
    L.fs_last_path.argtypes = []
    L.fs_last_path.restype = C.c_char_p
    if path == LIB_PATH:
        _lib = L
    return L


def _check(name: str, status: int) -> None:
    if status != 0:
        L = load()
        raise FsError(f"{name}: {L.fs_status_string(status).decode()}: "
                      f"{L.fs_last_error().decode()}", status)


def _p(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _s(stream):
    if stream is None:
        return C.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return C.c_void_p(stream.cuda_stream)
    return C.c_void_p(int(stream))


def _strides(t, default):
    if t is None:
        return default
    if t.dim() != 4 or t.stride(3) != 1:
        raise FsError("tensors must be [B, H, T, d] with d contiguous")
    return tuple(t.stride()[:3])


def problem(batch: int, heads: int, head_dim: int, n_ctx: int, n_q: int, q_pos0: int,
            window: int, dtype: int, cell: int = CELL, q=None, kv=None, o=None) -> FsProblem:
    """fs_problem for [B, H, T, d] tensors (contiguous unless tensors are given)."""
    dq = (heads * n_q * head_dim, n_q * head_dim, head_dim)
    dkv = (heads * n_ctx * head_dim, n_ctx * head_dim, head_dim)
    p = FsProblem()
    p.batch, p.heads, p.head_dim, p.n_ctx = batch, heads, head_dim, n_ctx
    p.n_q, p.q_pos0, p.cell, p.window, p.dtype, p.reserved = n_q, q_pos0, cell, window, dtype, 0
    p.q_stride[:] = _strides(q, dq)
    p.kv_stride[:] = _strides(kv, dkv)
    p.o_stride[:] = _strides(o, dq)
    return p


# ---- the C ABI, one wrapper per entry point ---------------------------------
def fs_cell_summaries(prob, k, kbar, amax, stream=None):
    _check("fs_cell_summaries", load().fs_cell_summaries(C.byref(prob), _p(k), _p(kbar),
                                                         _p(amax), _s(stream)))


def fs_prune_rows(prob):
    lo, rows = C.c_int32(), C.c_int32()
    _check("fs_prune_rows", load().fs_prune_rows(C.byref(prob), C.byref(lo), C.byref(rows)))
    return lo.value, rows.value


def fs_prune_workspace_size(prob) -> int:
    n = C.c_size_t()
    _check("fs_prune_workspace_size", load().fs_prune_workspace_size(C.byref(prob), C.byref(n)))
    return n.value


def fs_prune_prefix(prob, amax, n_recent, budget, keep, keep_count, stream=None, workspace=None):
    """workspace: None, or a device buffer of >= fs_prune_workspace_size bytes."""
    ws, nbytes = (None, 0) if workspace is None else \
        (_p(workspace), workspace.numel() * workspace.element_size())
    _check("fs_prune_prefix", load().fs_prune_prefix(C.byref(prob), _p(amax), n_recent, budget,
                                                     _p(keep), _p(keep_count), ws, nbytes,
                                                     _s(stream)))


def fs_select_topk(prob, q, kbar, keep, keep_count, keep_width, topk, idx, score=None,
                   stream=None, prior=None, workspace=None):
    """prior: None, or (amax, lambda, sigma) device tensors for eq. 7's position prior;
    workspace: None, or a device buffer of >= fs_select_workspace_size bytes."""
    amax, lam, sig = prior if prior is not None else (None, None, None)
    ws, nbytes = (None, 0) if workspace is None else \
        (_p(workspace), workspace.numel() * workspace.element_size())
    _check("fs_select_topk", load().fs_select_topk(C.byref(prob), _p(q), _p(kbar), _p(amax),
                                                   _p(lam), _p(sig), _p(keep), _p(keep_count),
                                                   keep_width, topk, _p(idx), _p(score), ws,
                                                   nbytes, _s(stream)))


def fs_select_workspace_size(prob, keep_width, topk) -> int:
    """keep_width: the keep rows' width, 0 without pruning."""
    n = C.c_size_t()
    _check("fs_select_workspace_size",
           load().fs_select_workspace_size(C.byref(prob), int(keep_width), int(topk), C.byref(n)))
    return n.value


def fs_rerank_topk(prob, q, k, keep, keep_count, keep_width, topk, idx, score=None,
                   stream=None, prior=None, workspace=None):
    """Eq. 12 reranking + top-K; prior: None or (amax, lambda, sigma) device tensors;
    workspace: None, or a device buffer of >= fs_rerank_workspace_size bytes."""
    amax, lam, sig = prior if prior is not None else (None, None, None)
    ws, nbytes = (None, 0) if workspace is None else \
        (_p(workspace), workspace.numel() * workspace.element_size())
    _check("fs_rerank_topk", load().fs_rerank_topk(C.byref(prob), _p(q), _p(k), _p(amax), _p(lam),
                                                   _p(sig), _p(keep), _p(keep_count), keep_width,
                                                   topk, _p(idx), _p(score), ws, nbytes,
                                                   _s(stream)))


def fs_rerank_workspace_size(prob, keep_width) -> int:
    """keep_width: the keep rows' width, 0 without pruning."""
    n = C.c_size_t()
    _check("fs_rerank_workspace_size",
           load().fs_rerank_workspace_size(C.byref(prob), int(keep_width), C.byref(n)))
    return n.value


def fs_forest_size(prob) -> int:
    """Bytes of one FS-B forest (every (b, h)) for this problem's shape."""
    n = C.c_size_t()
    _check("fs_forest_size", load().fs_forest_size(C.byref(prob), C.byref(n)))
    return n.value


def fs_forest_build(prob, kbar, amax, forest, tau=None, stream=None):
    """FS-B forest (eq. 10) into `forest` (a device buffer of fs_forest_size bytes,
    256-byte aligned): every cell when tau is None, else the cells with amax >= tau[h]."""
    _check("fs_forest_build", load().fs_forest_build(C.byref(prob), _p(kbar), _p(amax), _p(tau),
                                                     _p(forest), _s(stream)))


def fs_beam_select(prob, q, forest0, forest_tau, beam, slack, topk, idx, score=None,
                   prior=None, effort=None, stream=None, k=None):
    """FS-B beam search (eq. 11) for S_i; prior: None or (lambda, sigma) device tensors;
    effort: None or an int32 [B, H, n_q] tensor for the node scores per query;
    k: None (rank the found cells by eq. 7) or the raw keys (rank them by eq. 12)."""
    lam, sig = prior if prior is not None else (None, None)
    _check("fs_beam_select", load().fs_beam_select(C.byref(prob), _p(q), _p(k), _p(forest0),
                                                   _p(forest_tau), int(beam), float(slack),
                                                   _p(lam), _p(sig), int(topk), _p(idx),
                                                   _p(score), _p(effort), _s(stream)))


def fs_workspace_size(prob) -> int:
    n = C.c_size_t()
    _check("fs_workspace_size", load().fs_workspace_size(C.byref(prob), C.byref(n)))
    return n.value


def fs_window_attn(prob, q, k, v, rope_base, workspace, o_sr, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check("fs_window_attn", load().fs_window_attn(C.byref(prob), _p(q), _p(k), _p(v),
                                                   float(rope_base), _p(workspace), nbytes,
                                                   _p(o_sr), _s(stream)))


def fs_window_table(prob, rope_base, workspace, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check("fs_window_table", load().fs_window_table(C.byref(prob), float(rope_base),
                                                     _p(workspace), nbytes, _s(stream)))


def fs_window_attn_tabled(prob, q, k, v, workspace, o_sr, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check("fs_window_attn_tabled",
           load().fs_window_attn_tabled(C.byref(prob), _p(q), _p(k), _p(v), _p(workspace),
                                        nbytes, _p(o_sr), _s(stream)))


def fs_sparse_workspace_size(prob) -> int:
    n = C.c_size_t()
    _check("fs_sparse_workspace_size", load().fs_sparse_workspace_size(C.byref(prob), C.byref(n)))
    return n.value


def fs_sparse_attn(prob, q, k, v, idx, topk, rms_eps, o_lr, workspace=None, stream=None):
    """workspace: None (unsplit) or a device buffer of >= fs_sparse_workspace_size bytes."""
    ws, nbytes = (None, 0) if workspace is None else \
        (_p(workspace), workspace.numel() * workspace.element_size())
    _check("fs_sparse_attn", load().fs_sparse_attn(C.byref(prob), _p(q), _p(k), _p(v), _p(idx),
                                                   topk, float(rms_eps), ws, nbytes, _p(o_lr),
                                                   _s(stream)))


def last_path() -> str:
    """The kernel path of the calling thread's last readout / window / selection call."""
    return load().fs_last_path().decode()


def fs_sparse_attn_combine(prob, q, k, v, idx, topk, rms_eps, o_sr, alpha, o, workspace=None,
                           stream=None):
    """Eq. 9's readout with eq. 2 in its epilogue: o = o_sr + alpha_h * o_lr (o may be o_sr)."""
    ws, nbytes = (None, 0) if workspace is None else \
        (_p(workspace), workspace.numel() * workspace.element_size())
    _check("fs_sparse_attn_combine",
           load().fs_sparse_attn_combine(C.byref(prob), _p(q), _p(k), _p(v), _p(idx), topk,
                                         float(rms_eps), _p(o_sr), _p(alpha), ws, nbytes, _p(o),
                                         _s(stream)))


def fs_sparse_attn_noalloc(prob, q, k, v, idx, topk, rms_eps, o_lr, stream=None):
    """fs_sparse_attn with the split states in the library's own device array (no
    workspace, no allocation)."""
    _check("fs_sparse_attn_noalloc",
           load().fs_sparse_attn_noalloc(C.byref(prob), _p(q), _p(k), _p(v), _p(idx), topk,
                                         float(rms_eps), _p(o_lr), _s(stream)))


def fs_combine(prob, o_sr, o_lr, alpha, o, stream=None):
    _check("fs_combine", load().fs_combine(C.byref(prob), _p(o_sr), _p(o_lr), _p(alpha), _p(o),
                                           _s(stream)))


# ---- the whole forward: buffers allocated once, six calls per step -----------
class FsForward:
    """The FS-L forward of one problem shape: eq. 5, 8, 7, 3-4, 9, then 2.

    All intermediates are allocated at construction; a call enqueues the six
    library calls on the stream and allocates nothing.  The window's RoPE table
    depends only on (w, d, rope_base): the first call builds it in the workspace,
    later calls reuse it (fs_window_attn_tabled)."""

    def __init__(self, batch, heads, n_ctx, head_dim, n_q, q_pos0, dtype, topk, budget,
                 n_recent=0, window=512, rope_base=10000.0, rms_eps=1e-6, device="cuda",
                 prior_lambda=None, prior_sigma=None):
        self.dtype = FS_BF16 if dtype in ("bf16", torch.bfloat16, FS_BF16) else FS_F32
        tdt = torch.bfloat16 if self.dtype == FS_BF16 else torch.float32
        self.prob = problem(batch, heads, head_dim, n_ctx, n_q, q_pos0, window, self.dtype)
        self.topk, self.budget, self.n_recent = topk, budget, n_recent
        self.rope_base, self.rms_eps = rope_base, rms_eps
        n_cells = n_ctx // CELL
        B, H, d = batch, heads, head_dim
        self.n_lo, self.n_rows = fs_prune_rows(self.prob)
        f32, i32 = torch.float32, torch.int32
        self.kbar = torch.empty((B, H, max(n_cells, 1), d), dtype=f32, device=device)
        self.amax = torch.empty((B, H, max(n_cells, 1)), dtype=f32, device=device)
        self.pruned = budget >= 0
        self.keep_w = n_recent + budget if self.pruned else 0
        self.keep = self.keep_count = None
        if self.pruned:
            self.keep = torch.empty((B, H, max(self.n_rows, 1), self.keep_w), dtype=i32,
                                    device=device)
            self.keep_count = torch.empty((B, H, max(self.n_rows, 1)), dtype=i32, device=device)
        self.idx = torch.empty((B, H, n_q, topk), dtype=i32, device=device)
        self.score = torch.empty((B, H, n_q, topk), dtype=f32, device=device)
        self.ws = torch.empty(fs_workspace_size(self.prob), dtype=torch.uint8, device=device)
        self.table_ready = False
        npr = fs_prune_workspace_size(self.prob) if self.pruned else 0
        self.ws_prune = torch.empty(npr, dtype=torch.uint8, device=device) if npr else None
        nsp = fs_sparse_workspace_size(self.prob)
        self.ws_sparse = torch.empty(nsp, dtype=torch.uint8, device=device) if nsp else None
        nsel = fs_select_workspace_size(self.prob, self.keep_w, topk)
        self.ws_select = torch.empty(nsel, dtype=torch.uint8, device=device) if nsel else None
        self.o_sr = torch.empty((B, H, n_q, d), dtype=tdt, device=device)
        self.o_lr = torch.empty_like(self.o_sr)
        self.o = torch.empty_like(self.o_sr)
        # eq. 7's position prior: per-head lambda / sigma (float32), or none
        self.prior = None
        if prior_lambda is not None:
            lam = torch.as_tensor(prior_lambda, dtype=f32).to(device)
            sig = torch.as_tensor(prior_sigma, dtype=f32).to(device)
            assert lam.shape == (H,) and sig.shape == (H,)
            self.prior = (self.amax, lam, sig)

    def __call__(self, q, k, v, alpha, stream=None, keep_score=True, fused=False):
        """The forward; fused: eq. 2 in the readout's epilogue (fs_sparse_attn_combine),
        so o_lr is not written."""
        p = self.prob
        fs_cell_summaries(p, k, self.kbar, self.amax, stream)
        if self.pruned:
            fs_prune_prefix(p, self.amax, self.n_recent, self.budget, self.keep, self.keep_count,
                            stream, self.ws_prune)
        fs_select_topk(p, q, self.kbar, self.keep, self.keep_count, self.keep_w, self.topk,
                       self.idx, self.score if keep_score else None, stream, self.prior,
                       self.ws_select)
        if self.table_ready:
            fs_window_attn_tabled(p, q, k, v, self.ws, self.o_sr, stream)
        else:
            fs_window_attn(p, q, k, v, self.rope_base, self.ws, self.o_sr, stream)
            # a build recorded into a graph under capture has not run yet
            self.table_ready = not torch.cuda.is_current_stream_capturing()
        if fused:
            fs_sparse_attn_combine(p, q, k, v, self.idx, self.topk, self.rms_eps, self.o_sr,
                                   alpha, self.o, self.ws_sparse, stream)
            return self.o
        fs_sparse_attn(p, q, k, v, self.idx, self.topk, self.rms_eps, self.o_lr, self.ws_sparse,
                       stream)
        fs_combine(p, self.o_sr, self.o_lr, alpha, self.o, stream)
        return self.o

    @classmethod
    def for_workload(cls, wl, device="cuda"):
        lam, sig = wl.prior_arrays() if hasattr(wl, "prior_arrays") else (None, None)
        return cls(wl.batch, wl.heads, wl.n_ctx, wl.head_dim, wl.n_q, wl.q_pos0, wl.dtype,
                   wl.topk, wl.budget, wl.n_recent, wl.window, wl.rope_base, wl.rms_eps, device,
                   lam, sig)


# ---- streaming FS-L: a bounded per-head state --------------------------------------
class FsbSelect:
    """FS-B selection (section 3.4) for one problem shape: both forests' storage
    and the outputs are allocated at construction; build() enqueues the two
    forest builds (eq. 10) from the cell summaries, select() the beam search
    (eq. 11).  The forests depend on the cells only, so one build serves any
    query range over the same keys (pass that range's problem to select)."""

    def __init__(self, prob, topk, beam=32, slack=1.0, admitted=True, device="cuda"):
        self.prob, self.topk, self.beam, self.slack = prob, topk, beam, slack
        nb = fs_forest_size(prob)
        self.forest0 = torch.empty(nb, dtype=torch.uint8, device=device)
        self.forest_tau = torch.empty(nb, dtype=torch.uint8, device=device) if admitted else None
        B, H, nq = prob.batch, prob.heads, prob.n_q
        self.idx = torch.empty((B, H, nq, topk), dtype=torch.int32, device=device)
        self.score = torch.empty((B, H, nq, topk), dtype=torch.float32, device=device)
        self.effort = torch.empty((B, H, nq), dtype=torch.int32, device=device)

    def build(self, kbar, amax, tau=None, stream=None):
        """kbar, amax: eq. 5 summaries (as fs_cell_summaries writes them); tau: the
        admitted forest's float32 [H] thresholds (required when it was allocated)."""
        fs_forest_build(self.prob, kbar, amax, self.forest0, stream=stream)
        if self.forest_tau is not None:
            if tau is None:
                raise FsError("FsbSelect.build: the admitted forest needs tau")
            fs_forest_build(self.prob, kbar, amax, self.forest_tau, tau=tau, stream=stream)

    def select(self, q, prob=None, idx=None, score=False, effort=False, prior=None,
               stream=None, k=None):
        """S_i into self.idx (or `idx`, for another query range's problem `prob`).
        score / effort: False (not written), True (into self.score / self.effort)
        or a tensor; prior: None or (lambda, sigma) device tensors; k: None, or the
        raw keys to rank the found cells by eq. 12 instead of eq. 7.  Returns idx."""
        p = prob or self.prob
        mine = self.prob
        if prob is not None:
            same = all(getattr(prob, f) == getattr(mine, f)
                       for f in ("batch", "heads", "head_dim", "n_ctx", "cell", "dtype"))
            if not same:
                raise FsError("FsbSelect.select: prob must match the forests' batch, heads, "
                              "head_dim, n_ctx, cell and dtype")
        B, H, nq = p.batch, p.heads, p.n_q
        if nq != mine.n_q and (idx is None or score is True or effort is True):
            raise FsError("FsbSelect.select: a query range of another length needs its own "
                          "idx (and score / effort tensors)")
        out = self.idx if idx is None else idx
        sc = self.score if score is True else (score if score is not False else None)
        ef = self.effort if effort is True else (effort if effort is not False else None)
        for name, t, shape in (("idx", out, (B, H, nq, self.topk)),
                               ("score", sc, (B, H, nq, self.topk)), ("effort", ef, (B, H, nq))):
            if t is not None and tuple(t.shape) != shape:
                raise FsError(f"FsbSelect.select: {name} has shape {tuple(t.shape)}, "
                              f"expected {shape}")
        fs_beam_select(p, q, self.forest0, self.forest_tau, self.beam, self.slack, self.topk,
                       out, sc, prior=prior, effort=ef, stream=stream, k=k)
        return out


def fs_stream_state_size(cfg: FsStreamConfig) -> int:
    n = C.c_size_t()
    _check("fs_stream_state_size", load().fs_stream_state_size(C.byref(cfg), C.byref(n)))
    return n.value


def fs_stream_reset(cfg: FsStreamConfig, state, stream=None):
    _check("fs_stream_reset", load().fs_stream_reset(C.byref(cfg), _p(state),
                                                      state.numel() * state.element_size(),
                                                      _s(stream)))


def fs_stream_step(cfg: FsStreamConfig, state, pos0: int, q, k, v, alpha, o, idx=None,
                   prior=None, stream=None):
    """Append k, v ([B, H, n_new, d], contiguous) at positions pos0 .. and write the
    FS-L output of the queries q at those positions into o; prior: None or
    (lambda, sigma) float32 [H] device tensors; idx: optional selected cells."""
    lam, sig = prior if prior is not None else (None, None)
    _check("fs_stream_step", load().fs_stream_step(
        C.byref(cfg), _p(state), state.numel() * state.element_size(), int(pos0),
        int(q.shape[2]), _p(q), _p(k), _p(v), _p(alpha), _p(lam), _p(sig), _p(o), _p(idx),
        _s(stream)))


class FsStream:
    """A streaming FS-L layer state on one device: `step(q, k, v)` appends the
    tokens and returns their outputs, reading only the fixed-size state."""

    def __init__(self, batch, heads, head_dim, window, n_recent, budget, topk, max_new,
                 dtype, alpha, rope_base=10000.0, rms_eps=1e-6, prior_lambda=None,
                 prior_sigma=None, device="cuda"):
        self.cfg = FsStreamConfig(batch, heads, head_dim, CELL, window, n_recent, budget, topk,
                                  max_new, dtype, rope_base, rms_eps)
        self.bytes = fs_stream_state_size(self.cfg)
        self.state = torch.empty(self.bytes, dtype=torch.uint8, device=device)
        self.alpha = alpha
        self.prior = None if prior_lambda is None else (prior_lambda, prior_sigma)
        self.pos = 0
        fs_stream_reset(self.cfg, self.state)

    def reset(self):
        fs_stream_reset(self.cfg, self.state)
        self.pos = 0

    def step(self, q, k, v, o=None, idx=None):
        if o is None:
            o = torch.empty_like(q)
        fs_stream_step(self.cfg, self.state, self.pos, q, k, v, self.alpha, o, idx, self.prior)
        self.pos += q.shape[2]
        return o

