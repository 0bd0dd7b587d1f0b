"""The forward captured in a HIP graph (torch.cuda.CUDAGraph over the C-ABI
calls; the library makes no allocation, copy or memset, so every call
captures) replays to the eager result bit for bit: three replays with eager
work and synchronisations between them, on a prefill with the MFMA kernels, a
short query range whose selection, window and readout split over workgroups
(workspaces), and fp32 storage (the fp32 matrix-core selection, window and
readout)."""
import numpy as np
import pytest

from long_context_fs_amd import synth

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from fs_testutil import to_dev  # noqa: E402
from long_context_fs_amd.fs import FsForward  # noqa: E402

W = synth.WORKLOADS
CASES = {
    "bf16_d128_prefill": W["prefill_b1h8_n65536_d128_bf16"].replace(
        heads=2, n_ctx=4100, n_q=4100, budget=24, topk=8),
    "bf16_d128_decode_split": W["decode_b1h8_n262144_q256_d128_bf16"].replace(
        heads=2, n_ctx=9000, n_q=77, q_pos0=9000 - 77, budget=200, topk=16, needle_queries=77),
    "f32_d64": W["prefill_b1h1_n2048_d64_f32"].replace(heads=2, n_ctx=1500, n_q=1500),
}


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("fused", [True, False])
def test_graph_replays_equal_eager(name, fused):
    wl = CASES[name]
    x = synth.generate(wl)
    q, k, v = (to_dev(x[n], wl.dtype) for n in ("q", "k", "v"))
    alpha = torch.from_numpy(x["alpha"]).cuda()
    fwd = FsForward.for_workload(wl)
    fwd(q, k, v, alpha, fused=fused)
    torch.cuda.synchronize()
    want_o, want_idx = _bits(fwd.o), fwd.idx.cpu().numpy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd(q, k, v, alpha, fused=fused)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd(q, k, v, alpha, fused=fused)
    torch.cuda.synchronize()
    for rep in range(3):
        fwd.o.fill_(float("nan"))
        fwd.idx.fill_(-7)
        noise = torch.randn(1 << 16, device="cuda")           # eager work between replays
        float((noise * noise).sum())
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(fwd.idx.cpu().numpy(), want_idx, err_msg=f"replay {rep}")
        np.testing.assert_array_equal(_bits(fwd.o), want_o, err_msg=f"replay {rep}")
