"""The C ABI on the host: the library loads, exports what include/fs.h declares,
and rejects bad arguments before enqueuing anything (no GPU is touched)."""
import ctypes as C
import os
import re
import subprocess

import pytest

from long_context_fs_amd import fs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fs.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fs_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fs.LIB_PATH):
        pytest.skip("libfs.so not built")
    return fs.load()


def test_header_declares_the_six_calls():
    names = _declared()
    for n in ("fs_cell_summaries", "fs_prune_prefix", "fs_select_topk", "fs_window_attn",
              "fs_sparse_attn", "fs_combine", "fs_rerank_topk", "fs_stream_step"):
        assert n in names
    assert set(names) == set(fs.SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", fs.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (fs_[a-z_]+)$", out, flags=re.M))
    for n in _declared():
        assert n in exported, n
        assert hasattr(lib, n)


def test_header_compiles_as_c():
    src = '#include "fs.h"\nint main(void){fs_problem p; (void)p; return (int)FS_OK;}\n'
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                        "-x", "c", "-", "-fsyntax-only"], input=src, text=True,
                       capture_output=True)
    assert r.returncode == 0, r.stderr


def _prob(**kw):
    f = dict(batch=1, heads=2, head_dim=64, n_ctx=4096, n_q=4096, q_pos0=0, window=512,
             dtype=fs.FS_BF16)
    f.update(kw)
    return fs.problem(**f)


FAKE = C.c_void_p(1 << 20)          # aligned, never dereferenced: validation fails first


def test_prune_rows_and_workspace_host_only(lib):
    assert fs.fs_prune_rows(_prob()) == (0, 112)          # n = (4095-512)//32 = 111
    assert fs.fs_prune_rows(_prob(n_q=256, q_pos0=4096 - 256)) == ((3840 - 512) // 32, 8)
    assert fs.fs_prune_rows(_prob(n_q=0)) == (0, 0)
    assert fs.fs_prune_rows(_prob(n_q=100, n_ctx=400)) == (0, 1)
    ws = fs.fs_workspace_size(_prob())
    table = (512 + 256) * 32 * 8                           # (w + 256) x d/2 float2
    # 2 x 32 query tiles fill 64 < 512 workgroups: each tile's keys split 8 ways,
    # one partial (O row of d floats, then (m, l)) per query and split
    assert ws == table + 2 * 4096 * 8 * (64 * 4 + 8)
    # enough queries to fill the device: the table alone
    assert fs.fs_workspace_size(_prob(batch=8, heads=16, n_q=4096)) == table
    # selection splits a short query range's union over 64-cell workgroups: 256
    # queries of 2 heads, keep rows of 500 cells -> union up to 503 -> 512 slots, 8 splits
    dec = _prob(n_ctx=65536, n_q=256, q_pos0=65536 - 256)
    assert fs.fs_select_workspace_size(dec, 500, 32) == 2 * 256 * 8 * 32 * 8
    assert fs.fs_select_workspace_size(dec, 40, 32) == 0           # union of 48 slots
    assert fs.fs_select_workspace_size(_prob(batch=8, heads=16), 500, 32) == 0   # 2048 tiles
    # fp32 storage splits alike
    assert fs.fs_select_workspace_size(_prob(dtype=fs.FS_F32, n_ctx=65536, n_q=256,
                                             q_pos0=65536 - 256), 500, 32) == 2 * 256 * 8 * 32 * 8


def test_readout_split_states_bounded(lib):
    """The readout splits a short query range into at most 256 workgroups of 128
    query rows (one per CU), each row's state d fp32 plus (m, l); so no shape's
    states exceed 256 x 128 x 520 bytes, the allocation-free readout's array,
    and the 256k decode shape (8 heads x 2 tiles, 16 splits) fills it."""
    cap = 256 * 128 * (128 * 4 + 8)
    worst = 0
    for heads in (1, 2, 3, 5, 8, 16, 17, 40, 100, 255, 256, 300):
        for n_q in (1, 77, 128, 129, 256, 300, 1000, 4096):
            for d in (64, 128):
                p = _prob(heads=heads, head_dim=d, n_ctx=8192, n_q=n_q, q_pos0=8192 - n_q)
                need = fs.fs_sparse_workspace_size(p)
                tiles = (n_q + 127) // 128 * heads
                splits = min(32, 256 // tiles) if tiles <= 256 else 1
                rows = heads * n_q
                assert need == (0 if splits <= 1 else rows * splits * (d * 4 + 8)), (heads, n_q, d)
                worst = max(worst, need)
    assert worst <= cap
    dec = _prob(heads=8, head_dim=128, n_ctx=262144, n_q=256, q_pos0=262144 - 256)
    assert fs.fs_sparse_workspace_size(dec) == cap


@pytest.mark.parametrize("bad,status", [
    (dict(head_dim=96), 2), (dict(head_dim=0), 2), (dict(cell=16), 2), (dict(batch=0), 1),
    (dict(n_ctx=0), 1), (dict(n_q=10, q_pos0=4090), 1), (dict(window=-1), 2),
    (dict(dtype=7), 1),
])
def test_invalid_problem_rejected(lib, bad, status):
    p = _prob(**bad)
    with pytest.raises(fs.FsError) as e:
        fs.fs_prune_rows(p)
    assert e.value.status == status


def test_bad_strides_and_pointers_rejected(lib):
    p = _prob()
    p.q_stride[2] = 60                                    # rows not 16-byte aligned
    st = lib.fs_cell_summaries(C.byref(p), FAKE, FAKE, FAKE, None)
    assert st == 1 and b"q_stride" in lib.fs_last_error()
    p = _prob()
    assert lib.fs_cell_summaries(C.byref(p), None, FAKE, FAKE, None) == 1
    assert b"k is NULL" in lib.fs_last_error()
    assert lib.fs_cell_summaries(C.byref(p), C.c_void_p((1 << 20) + 4), FAKE, FAKE, None) == 1
    assert b"aligned" in lib.fs_last_error()
    assert lib.fs_cell_summaries(None, FAKE, FAKE, FAKE, None) == 1


def test_call_specific_limits(lib):
    p = _prob()
    assert lib.fs_prune_prefix(C.byref(p), FAKE, 0, 0, FAKE, FAKE, None, 0, None) == 2
    assert lib.fs_prune_prefix(C.byref(p), FAKE, 0, 5000, FAKE, FAKE, None, 0, None) == 2
    assert lib.fs_prune_prefix(C.byref(p), FAKE, -1, 4, FAKE, FAKE, None, 0, None) == 2
    # an undersized prune workspace is an error; the size is one int32 per (b, h) and cell
    # below the largest candidate count (4096 tokens, w 512: 111 cells, 2 heads)
    assert fs.fs_prune_workspace_size(p) == 2 * 111 * 4
    assert lib.fs_prune_prefix(C.byref(p), FAKE, 0, 8, FAKE, FAKE, FAKE, 16, None) == 1
    assert b"workspace" in lib.fs_last_error()
    assert lib.fs_select_topk(C.byref(p), FAKE, FAKE, None, None, None, None, None, 0, 0, FAKE,
                              None, None, 0, None) == 2
    assert lib.fs_select_topk(C.byref(p), FAKE, FAKE, None, None, None, None, None, 0, 65, FAKE,
                              None, None, 0, None) == 2
    assert lib.fs_select_topk(C.byref(p), FAKE, FAKE, None, None, None, FAKE, None, 64, 8, FAKE,
                              None, None, 0, None) == 1
    # the prior needs all three of amax, lambda and sigma
    assert lib.fs_select_topk(C.byref(p), FAKE, FAKE, None, FAKE, FAKE, None, None, 0, 8, FAKE,
                              None, None, 0, None) == 1
    assert b"prior" in lib.fs_last_error()
    assert lib.fs_select_topk(C.byref(p), FAKE, FAKE, FAKE, FAKE, None, None, None, 0, 8, FAKE,
                              None, None, 0, None) == 1
    assert lib.fs_select_topk(C.byref(p), FAKE, FAKE, None, None, None, None, None, 0, 8, FAKE,
                              None, C.c_void_p(0x1010), 1 << 20, None) == 1
    assert b"aligned" in lib.fs_last_error()
    sw = C.c_size_t()
    assert lib.fs_select_workspace_size(C.byref(p), 0, 0, C.byref(sw)) == 2
    assert lib.fs_select_workspace_size(C.byref(p), -1, 8, C.byref(sw)) == 1
    assert lib.fs_sparse_attn(C.byref(p), FAKE, FAKE, FAKE, None, 8, 1e-6, None, 0, FAKE,
                              None) == 1
    assert lib.fs_sparse_attn(C.byref(p), FAKE, FAKE, FAKE, FAKE, 8, -1.0, None, 0, FAKE,
                              None) == 1
    need = C.c_size_t()
    assert lib.fs_sparse_workspace_size(C.byref(p), C.byref(need)) == 0
    if need.value > 0:    # an undersized workspace is an error, not a silent fallback
        assert lib.fs_sparse_attn(C.byref(p), FAKE, FAKE, FAKE, FAKE, 8, 1e-6, FAKE, 16, FAKE,
                                  None) == 1
        assert b"workspace" in lib.fs_last_error()
    # the readout with eq. 2 in its epilogue needs o_sr, alpha and o
    assert lib.fs_sparse_attn_combine(C.byref(p), FAKE, FAKE, FAKE, FAKE, 8, 1e-6, None, FAKE,
                                      None, 0, FAKE, None) == 1
    assert lib.fs_sparse_attn_combine(C.byref(p), FAKE, FAKE, FAKE, FAKE, 8, 1e-6, FAKE, None,
                                      None, 0, FAKE, None) == 1
    assert b"alpha" in lib.fs_last_error()
    assert lib.fs_sparse_attn_combine(C.byref(p), FAKE, FAKE, FAKE, FAKE, 65, 1e-6, FAKE, FAKE,
                                      None, 0, FAKE, None) == 2
    # reranking validates like selection, and needs the keys
    assert lib.fs_rerank_topk(C.byref(p), FAKE, None, None, None, None, None, None, 0, 8, FAKE,
                              None, None, 0, None) == 1
    assert lib.fs_rerank_topk(C.byref(p), FAKE, FAKE, None, None, None, None, None, 0, 65, FAKE,
                              None, None, 0, None) == 2
    assert lib.fs_rerank_topk(C.byref(p), FAKE, FAKE, None, FAKE, FAKE, None, None, 0, 8, FAKE,
                              None, None, 0, None) == 1
    assert lib.fs_rerank_topk(C.byref(p), FAKE, FAKE, None, None, None, None, None, 0, 8, FAKE,
                              None, C.c_void_p(0x1008), 1 << 20, None) == 1
    assert b"aligned" in lib.fs_last_error()
    rw = C.c_size_t()
    assert lib.fs_rerank_workspace_size(C.byref(p), -1, C.byref(rw)) == 1
    assert lib.fs_rerank_workspace_size(C.byref(p), 0, None) == 1
    assert lib.fs_window_attn(C.byref(p), FAKE, FAKE, FAKE, 10000.0, FAKE, 16, FAKE, None) == 1
    assert b"workspace" in lib.fs_last_error()
    assert lib.fs_window_attn(C.byref(p), FAKE, FAKE, FAKE, 0.5, FAKE, 1 << 30, FAKE, None) == 1
    # the table alone, and the window with a table already built
    assert lib.fs_window_table(C.byref(p), 10000.0, FAKE, 16, None) == 1
    assert b"workspace" in lib.fs_last_error()
    assert lib.fs_window_table(C.byref(p), 1.0, FAKE, 1 << 30, None) == 1
    assert lib.fs_window_table(C.byref(p), 10000.0, None, 1 << 30, None) == 1
    assert lib.fs_window_attn_tabled(C.byref(p), FAKE, FAKE, FAKE, FAKE, 16, FAKE, None) == 1
    assert b"workspace" in lib.fs_last_error()
    assert lib.fs_window_attn_tabled(C.byref(p), FAKE, None, FAKE, FAKE, 1 << 30, FAKE, None) == 1
    assert lib.fs_combine(C.byref(p), FAKE, FAKE, None, FAKE, None) == 1
    big = _prob(n_ctx=1 << 20, n_q=1 << 20)              # 32752 candidate cells, no pruning
    assert lib.fs_select_topk(C.byref(big), FAKE, FAKE, None, None, None, None, None, 0, 8, FAKE,
                              None, None, 0, None) == 2


def test_status_strings(lib):
    assert lib.fs_status_string(0) == b"FS_OK"
    assert lib.fs_status_string(3) == b"FS_ERR_HIP"


def _scfg(**kw):
    f = dict(batch=1, heads=8, head_dim=128, cell=32, window=512, n_recent=0, budget=512,
             topk=32, max_new=256, dtype=fs.FS_BF16, rope_base=10000.0, rms_eps=1e-6)
    f.update(kw)
    return fs.FsStreamConfig(*[f[n] for n, _ in fs.FsStreamConfig._fields_])


def test_stream_state_is_bounded(lib):
    """The streaming state is sized by the config alone (no sequence length enters the
    call) and, at the 256k decode shape, is a small fraction of the K/V it replaces."""
    n = fs.fs_stream_state_size(_scfg())
    kv_256k = 2 * 8 * 262144 * 128 * 2
    assert n < kv_256k / 8
    # the token-state terms of the page's bound, (P + W) s + w + B + s rows of K and V
    rows = (512 + 0 + 256 // 32 + 2) * 32 + 2 * 1024
    assert n >= 8 * rows * 128 * 2 * 2
    assert fs.fs_stream_state_size(_scfg(budget=1024)) > n > fs.fs_stream_state_size(_scfg(budget=64))


@pytest.mark.parametrize("bad, status", [
    (dict(head_dim=96), 2), (dict(cell=16), 2), (dict(n_recent=0, budget=0), 2),
    (dict(n_recent=24, budget=1001), 2), (dict(topk=65), 2), (dict(max_new=0), 2),
    (dict(max_new=4097), 2), (dict(dtype=7), 1), (dict(batch=0), 1), (dict(window=-1), 2),
    (dict(rope_base=1.0), 1), (dict(rms_eps=-1.0), 1)])
def test_stream_config_rejected(lib, bad, status):
    n = C.c_size_t()
    assert lib.fs_stream_state_size(C.byref(_scfg(**bad)), C.byref(n)) == status


def test_stream_step_arguments_rejected(lib):
    cfg = _scfg(max_new=16)
    need = fs.fs_stream_state_size(cfg)
    step = lambda state, size, pos0, n_new, lam=None, sig=None, q=FAKE: lib.fs_stream_step(  # noqa: E731
        C.byref(cfg), state, size, pos0, n_new, q, FAKE, FAKE, FAKE, lam, sig, FAKE, None, None)
    assert step(FAKE, need - 1, 0, 4) == 1                       # state too small
    assert step(C.c_void_p((1 << 20) + 16), need, 0, 4) == 1     # not 256-byte aligned
    assert step(None, need, 0, 4) == 1
    assert step(FAKE, need, 0, 0) == 1 and step(FAKE, need, 0, 17) == 1
    assert step(FAKE, need, -1, 4) == 2 and step(FAKE, need, (1 << 31) - 2, 4) == 2
    assert step(FAKE, need, 0, 4, lam=FAKE) == 1                 # prior arrays go together
    assert step(FAKE, need, 0, 4, q=C.c_void_p((1 << 20) + 2)) == 1
    assert lib.fs_stream_reset(C.byref(cfg), FAKE, need - 1, None) == 1


def test_fsb_arguments_rejected(lib):
    """FS-B calls validate on the host and launch nothing on error."""
    p = _prob()
    fs_ = C.c_size_t()
    assert lib.fs_forest_size(C.byref(p), C.byref(fs_)) == 0 and fs_.value > 0
    big = _prob(n_ctx=1 << 21, n_q=1)                    # 65536 cells
    assert lib.fs_forest_size(C.byref(big), C.byref(fs_)) == 2
    assert lib.fs_forest_size(C.byref(p), None) == 1
    F = C.c_void_p(1 << 20)                                # 256-byte aligned stand-in
    assert lib.fs_forest_build(C.byref(p), FAKE, FAKE, None, C.c_void_p((1 << 20) + 16),
                               None) == 1
    assert b"256-byte" in lib.fs_last_error()
    assert lib.fs_forest_build(C.byref(p), FAKE, None, None, F, None) == 1
    assert lib.fs_beam_select(C.byref(p), FAKE, None, None, None, 8, 1.0, None, None, 8, FAKE,
                              None, None, None) == 1
    assert lib.fs_beam_select(C.byref(p), FAKE, None, F, None, 0, 1.0, None, None, 8, FAKE, None,
                              None, None) == 2
    assert lib.fs_beam_select(C.byref(p), FAKE, None, F, None, 65, 1.0, None, None, 8, FAKE, None,
                              None, None) == 2
    assert lib.fs_beam_select(C.byref(p), FAKE, None, F, None, 8, -1.0, None, None, 8, FAKE, None,
                              None, None) == 1
    assert lib.fs_beam_select(C.byref(p), FAKE, None, F, None, 8, float("nan"), None, None, 8, FAKE,
                              None, None, None) == 1
    assert lib.fs_beam_select(C.byref(p), FAKE, None, F, None, 8, 1.0, FAKE, None, 8, FAKE, None,
                              None, None) == 1
    assert b"prior" in lib.fs_last_error()
    assert lib.fs_beam_select(C.byref(p), FAKE, None, F, None, 8, 1.0, None, None, 65, FAKE, None,
                              None, None) == 2
    assert lib.fs_beam_select(C.byref(p), FAKE, None, F, None, 8, 1.0, None, None, 8, None, None,
                              None, None) == 1
    # keys for eq. 12's reranking must keep 16-byte rows
    assert lib.fs_beam_select(C.byref(p), FAKE, C.c_void_p(FAKE.value + 2), F, None, 8, 1.0,
                              None, None, 8, FAKE, None, None, None) == 1
    assert b"k is not 16-byte aligned" in lib.fs_last_error()
    # forest storage grows with the number of cells and holds their node statistics
    small, large = C.c_size_t(), C.c_size_t()
    lib.fs_forest_size(C.byref(_prob(n_ctx=4096, n_q=1)), C.byref(small))
    lib.fs_forest_size(C.byref(_prob(n_ctx=8192, n_q=1)), C.byref(large))
    n_cells = 8192 // 32                                   # 2 heads, 2 n_cells - 1 nodes, d 64
    assert large.value > small.value >= 2 * (2 * n_cells // 2 - 1) * 64 * 4
    assert large.value >= 2 * (2 * n_cells - 1) * 64 * 4


def test_fsb_select_wrapper_checks_shapes(lib):
    """FsbSelect refuses a query range over other forests' cells, a range of another
    length without its own outputs, and outputs of the wrong shape, before any call
    (host tensors: nothing reaches the device)."""
    torch = pytest.importorskip("torch")
    p = _prob(n_ctx=2048, n_q=256, q_pos0=2048 - 256)
    sel = fs.FsbSelect(p, 8, beam=4, slack=1.0, device="cpu")
    q = torch.zeros((1, 2, 256, 64), dtype=torch.bfloat16)
    with pytest.raises(fs.FsError, match="must match"):
        sel.select(q, prob=_prob(n_ctx=4096, n_q=256, q_pos0=4096 - 256))
    with pytest.raises(fs.FsError, match="another length"):
        sel.select(q[:, :, :100], prob=_prob(n_ctx=2048, n_q=100, q_pos0=1000))
    bad = torch.zeros((1, 2, 100, 7), dtype=torch.int32)
    with pytest.raises(fs.FsError, match="idx has shape"):
        sel.select(q[:, :, :100], prob=_prob(n_ctx=2048, n_q=100, q_pos0=1000), idx=bad)
