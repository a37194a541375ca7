"""gspn4, the four-direction propagation as an autograd op: its gradients are
gspn_backward4's (bit for bit, through the C ABI), and they match the fp64
oracle's."""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_spatial_propagation_gspn_amd import gspn as G
from linear_spatial_propagation_gspn_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield
    torch.cuda.synchronize()


def _np(t):
    return t.detach().float().cpu().double().numpy()


@pytest.mark.parametrize("merge", [False, True])
@pytest.mark.parametrize("shape,shared,chunk", [((2, 3, 23, 41), False, 0), ((1, 3, 40, 72), True, 5)])
def test_gspn4_gradients(shape, shared, chunk, merge):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, "f32", shared, chunk, 123 + w)
    inp = make_inputs(wl, DEV)
    x = inp["x"].clone().requires_grad_(True)
    zs = [z.clone().requires_grad_(True) for z in inp["logits"]]
    ls = [l.clone().requires_grad_(True) for l in inp["lam"]]
    m = torch.randn((4, c), device=DEV).requires_grad_(True) if merge else None
    y = G.gspn4(x, zs, ls, chunk_len=chunk, merge=m)
    gy = torch.randn_like(y)
    grads = torch.autograd.grad(y, [x] + zs + ls + ([m] if merge else []), gy)
    torch.cuda.synchronize()
    ref = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk,
                           merge=m.detach() if merge else None)
    torch.cuda.synchronize()
    assert torch.equal(grads[0], ref[0])
    for d in range(4):
        assert torch.equal(grads[5 + d], ref[2][d])                  # dlam, deterministic
        assert torch.allclose(grads[1 + d], ref[1][d], rtol=1e-5, atol=1e-6)  # shared sums: fp32 atomics
    o = oracle.backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk=chunk,
                         merge=_np(m) if merge else None)
    assert oracle.normwise_error(_np(grads[0]), o[0]) <= 1e-5
    for d in range(4):
        assert oracle.normwise_error(_np(grads[5 + d]), o[1][d]) <= 1e-5
        assert oracle.normwise_error(_np(grads[1 + d]), o[2][d]) <= 1e-5
    if merge:
        assert oracle.normwise_error(_np(grads[9]), o[3]) <= 1e-5
    yo = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk, merge=_np(m) if merge else None)
    assert oracle.normwise_error(_np(y), yo) <= 1e-5
