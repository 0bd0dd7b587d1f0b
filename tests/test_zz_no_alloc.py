"""The allocation-free readout (fs_sparse_attn_noalloc, include/fs.h) against
fs_sparse_attn with a caller workspace: two calls in a row on the split
(decode) path, the second on a smaller problem, must give the same o_lr bit for
bit (the same kernels, splits and states, the states held in the library's
device array instead of the workspace), and the workspace path must match the
oracle's eq. 9 rows (FreeSolo summary, picx.dev page, section 3.3)."""
import numpy as np
import pytest

import oracle
from long_context_fs_amd import fs, synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _run(wl, seed):
    x = synth.generate(wl, seed)
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).cuda().to(dt) for n in ("q", "k", "v"))
    fwd = fs.FsForward.for_workload(wl)
    fwd(q, k, v, torch.from_numpy(x["alpha"]).cuda())
    assert fwd.ws_sparse is not None                   # the decode shape splits
    ref = torch.full_like(fwd.o_lr, float("nan"))
    fs.fs_sparse_attn(fwd.prob, q, k, v, fwd.idx, wl.topk, wl.rms_eps, ref, fwd.ws_sparse)
    got = torch.full_like(fwd.o_lr, float("nan"))
    fs.fs_sparse_attn_noalloc(fwd.prob, q, k, v, fwd.idx, wl.topk, wl.rms_eps, got)
    torch.cuda.synchronize()
    return x, fwd.idx.cpu().numpy(), ref.float().cpu().numpy(), got.float().cpu().numpy()


def test_noalloc_equals_workspace_twice():
    big = synth.WORKLOADS["decode_b1h8_n262144_q256_d128_bf16"].replace(
        n_ctx=65536, q_pos0=65536 - 256)
    small = big.replace(heads=2, n_ctx=20000, n_q=77, q_pos0=20000 - 77, needle_queries=77,
                        budget=96)
    for wl, seed in ((big, 5), (small, 6)):
        x, idx, ref, got = _run(wl, seed)
        assert np.isfinite(got).all()
        np.testing.assert_array_equal(got, ref)
        p = oracle.problem_from(wl)
        orc = oracle.Oracle()
        for h in range(wl.heads):
            for t in range(0, wl.n_q, 17):
                cells = idx[0, h, t][idx[0, h, t] >= 0]
                want = orc.sparse_row(p, x["q"][0, h, t], x["k"][0, h], x["v"][0, h], cells)
                err = np.abs(got[0, h, t] - want).max() / max(np.abs(want).max(), 1e-30)
                assert err <= 2e-2, (wl.n_ctx, h, t, err)


def test_noalloc_fp32_equals_workspace():
    """fp32 storage (the fp32 matrix-core readout and its split merge) through the
    allocation-free call: bit for bit the workspace call, and within the fp32
    tolerance of the oracle's eq. 9 rows."""
    wl = synth.WORKLOADS["decode_b1h8_n262144_q256_d128_bf16"].replace(
        dtype="f32", heads=4, n_ctx=20000, n_q=64, q_pos0=20000 - 64, needle_queries=64,
        budget=200)
    x, idx, ref, got = _run(wl, 7)
    assert np.isfinite(got).all()
    np.testing.assert_array_equal(got, ref)
    p = oracle.problem_from(wl)
    orc = oracle.Oracle()
    for h in range(wl.heads):
        for t in range(0, wl.n_q, 9):
            cells = idx[0, h, t][idx[0, h, t] >= 0]
            want = orc.sparse_row(p, x["q"][0, h, t], x["k"][0, h], x["v"][0, h], cells)
            err = np.abs(got[0, h, t] - want).max() / max(np.abs(want).max(), 1e-30)
            assert err <= 1e-4, (h, t, err)
