"""The library allocates nothing and issues only kernel launches on the
caller's stream (no memset, no synchronisation outside the *_timed calls),
so a forward or backward call can be captured in a HIP graph and replayed.
Each replay is checked against the eager result, with the program's own
eager work and synchronisations between replays."""
import sys

import pytest
import torch

from linear_spatial_propagation_gspn_amd import gspn as G
from linear_spatial_propagation_gspn_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield
    torch.cuda.synchronize()


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("shape,dtype,shared,kernel", [
    ((2, 3, 40, 56), "f32", False, "plane4_kernel"),
    ((1, 3, 40, 72), "bf16", True, "scan4lp_kernel"),
    ((1, 2, 520, 600), "bf16", True, "scan4band_kernel"),
])
def test_forward4_graph_replays(shape, dtype, shared, kernel):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, 0, 91 + w)
    _say("graph forward4 %s %s" % (shape, kernel))
    inp = make_inputs(wl, DEV)
    ws = G.forward4_workspace(inp["x"], wl.cw)
    m = torch.randn((4, c), device=DEV)
    ref, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], workspace=ws, merge=m)
    torch.cuda.synchronize()
    assert times["scan_kernel"] == kernel
    out = torch.empty_like(inp["x"])
    g = _capture(lambda: G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], out=out, workspace=ws, merge=m))
    for r in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), r
        junk = torch.randn(1 << 20, device=DEV).sum()  # eager work between replays
        torch.cuda.synchronize()
        del junk


@pytest.mark.parametrize("shape", [(1, 3, 40, 72), (2, 3, 30, 44)])   # long-line / plane-resident backward
def test_backward4_graph_replays(shape):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, "f32", True, 5, 93)
    inp = make_inputs(wl, DEV)
    gy = torch.randn(inp["x"].shape, device=DEV)
    ws = G.backward4_workspace(inp["x"], wl.cw)
    ref = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=5, workspace=ws)
    torch.cuda.synchronize()
    out = (torch.empty_like(inp["x"]), [torch.empty_like(z) for z in inp["logits"]],
           [torch.empty_like(l) for l in inp["lam"]])
    g = _capture(lambda: G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=5, workspace=ws,
                                          out=out))
    for r in range(3):
        out[0].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0], ref[0]), r
        for d in range(4):
            assert torch.equal(out[2][d], ref[2][d]), (r, d)
            # shared-logit sums are fp32 atomics: equal up to their order
            assert torch.allclose(out[1][d], ref[1][d], rtol=1e-5, atol=1e-6), (r, d)
