"""The allocation-free forward (gspn_forward4_noalloc, for callers that cannot
allocate device memory) through the C ABI, against the existing entry point
gspn_forward4 given a workspace of its own: the same kernels on the same
inputs, so the outputs must agree bit for bit, and with the fp64 oracle
within the usual normwise tolerances.  Two calls in a row, the second on a
smaller input, share the library's one static scratch array on the GPU."""
import sys

import pytest
import torch

import oracle
from linear_spatial_propagation_gspn_amd import gspn as G
from linear_spatial_propagation_gspn_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
DEV = "cuda"


def _np(t):
    return t.detach().float().cpu().double().numpy()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield
    torch.cuda.synchronize()


CALLS = [
    # a four-direction launch over long lines, with the learnable merge
    Workload("case", 2, 3, 300, 520, "f32", False, 0, 71),
    # then a smaller one: bf16, channel-shared weights (normalised into the scratch), chunks
    Workload("case", 1, 2, 100, 130, "bf16", True, 5, 72),
]


def test_noalloc_matches_the_workspace_forward():
    for i, wl in enumerate(CALLS):
        print("noalloc call %d: %s" % (i, (wl.n, wl.c, wl.h, wl.w, wl.dtype, wl.shared_w, wl.chunk)), flush=True)
        sys.stdout.flush()
        need = G.gspn_forward4_workspace_bytes(torch.empty(wl.n, wl.c, wl.h, wl.w, dtype=wl.torch_dtype), wl.cw)
        assert 0 < need <= G.NOALLOC_SCRATCH_BYTES
        inp = make_inputs(wl, DEV)
        m = torch.randn((4, wl.c), device=DEV) if i == 0 else None
        ref = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=wl.chunk,
                              workspace=G.forward4_workspace(inp["x"], wl.cw), merge=m)
        torch.cuda.synchronize()
        got = G.gspn_forward4_noalloc(inp["x"], inp["logits"], inp["lam"], chunk_len=wl.chunk, merge=m)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        o = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=wl.chunk,
                            merge=None if m is None else _np(m))
        assert oracle.normwise_error(_np(got), o) <= TOL[wl.dtype]


def test_noalloc_rejects_oversized_calls():
    x = torch.zeros(32, 1, 1024, 1024, device=DEV)
    zs = [torch.zeros(32, 1, 3, 1024, 1024, device=DEV) for _ in range(4)]
    with pytest.raises(G.GspnError) as e:
        G.gspn_forward4_noalloc(x, zs, [x] * 4)
    assert e.value.status == 11  # GSPN_ERR_WORKSPACE
