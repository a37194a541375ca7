"""GPU parity of the array layout (GSPN_LAYOUT_ARRAY): every direction's
logits as [N][Cw][3][H][W] and lambda as [N][C][H][W], the layout of the
boundary's statement of the problem.  The library copies the horizontal
directions' tensors into their scan frame (and the backward's horizontal
gradients back out), then runs the kernels of the scan layout, so the results
must equal the scan layout's bit for bit (up to the order of the fp32 atomics
that sum shared-logit gradients), and the oracle within the usual normwise
tolerances.  The oracle takes the scan layout: the tests transpose the
horizontal tensors to build the array-layout inputs."""
import sys

import numpy as np
import pytest
import torch

import oracle
from linear_spatial_propagation_gspn_amd import gspn as G
from linear_spatial_propagation_gspn_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _np(t):
    return t.detach().float().cpu().double().numpy()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield
    torch.cuda.synchronize()


def _array(ts):
    """Per-direction tensors from the scan frame to the array frame."""
    return [t if d < 2 else t.transpose(-1, -2).contiguous() for d, t in enumerate(ts)]


def _scan(ts):
    """Per-direction tensors from the array frame back to the scan frame."""
    return _array(ts)  # the transpose is its own inverse


def _gy(wl, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn((wl.n, wl.c_scan, wl.h, wl.w), generator=g, device=DEV,
                       dtype=torch.float32).to(wl.torch_dtype)


CASES = [
    ((1, 2, 16, 16), False),
    ((2, 3, 37, 70), False),     # rectangular: the horizontal frames differ in shape
    ((1, 2, 70, 37), True),
    ((1, 3, 40, 72), True),
    ((1, 2, 96, 80), False),     # larger than the plane-resident limit: the four-direction launch
    ((1, 2, 3, 1000), True),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [0, 5])
@pytest.mark.parametrize("shape,shared", CASES)
def test_forward4_array_layout(shape, shared, chunk, dtype):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 900 + h + w)
    _say("array layout forward %s shared=%s chunk=%d %s" % (shape, shared, chunk, dtype))
    inp = make_inputs(wl, DEV)
    za, la = _array(inp["logits"]), _array(inp["lam"])
    ya, times = G.gspn_forward4_timed(inp["x"], za, la, chunk_len=chunk,
                                      workspace=G.forward4_workspace(inp["x"], wl.cw, "array"), layout="array")
    ys = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk,
                         workspace=G.forward4_workspace(inp["x"], wl.cw))
    torch.cuda.synchronize()
    # two horizontal directions, logits and lambda each
    assert times["layout"]["launches"] == 4
    assert torch.equal(ya, ys)
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk)
    assert oracle.normwise_error(_np(ya), ref) <= TOL[dtype]


def test_forward4_array_layout_needs_workspace():
    wl = Workload("case", 1, 2, 16, 16, "f32", False, 0, 3)
    inp = make_inputs(wl, DEV)
    with pytest.raises(G.GspnError) as e:
        G.gspn_forward4(inp["x"], _array(inp["logits"]), _array(inp["lam"]), layout="array")
    assert e.value.status == 11  # GSPN_ERR_WORKSPACE


def test_forward4_array_layout_shared_lambda():
    """One lambda buffer for all four directions (allowed by the boundary):
    in the array layout it is the same array-frame tensor for every
    direction, copied once for the horizontal ones."""
    wl = Workload("case", 1, 3, 48, 80, "f32", False, 0, 21)
    inp = make_inputs(wl, DEV)
    lam = inp["lam"][0]  # [N][C][H][W]: the array frame
    ya, times = G.gspn_forward4_timed(inp["x"], _array(inp["logits"]), [lam] * 4,
                                      workspace=G.forward4_workspace(inp["x"], wl.cw, "array"), layout="array")
    torch.cuda.synchronize()
    assert times["layout"]["launches"] == 3  # two logit copies, one lambda copy
    lam_scan = [lam, lam, lam.transpose(-1, -2).contiguous(), lam.transpose(-1, -2).contiguous()]
    ref = oracle.forward4(inp["x"], inp["logits"], lam_scan)
    assert oracle.normwise_error(_np(ya), ref) <= TOL["f32"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_proxy_forward4_array_layout(dtype):
    wl = Workload("case", 1, 24, 40, 72, dtype, True, 0, 33, c_proxy=4)
    inp = make_inputs(wl, DEV)
    ya = G.gspn_proxy_forward4(inp["x"], inp["w_down"], inp["w_up"], _array(inp["logits"]), _array(inp["lam"]),
                               layout="array")
    ys = G.gspn_proxy_forward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"])
    torch.cuda.synchronize()
    assert torch.equal(ya, ys)
    ref = oracle.proxy_forward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"])
    assert oracle.normwise_error(_np(ya), ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [0, 5])
@pytest.mark.parametrize("shape,shared", CASES)
def test_backward4_array_layout(shape, shared, chunk, dtype):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 950 + h + w)
    _say("array layout backward %s shared=%s chunk=%d %s" % (shape, shared, chunk, dtype))
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 41)
    t = G.StageTimes()
    dxa, dza, dla = G.gspn_backward4(inp["x"], _array(inp["logits"]), _array(inp["lam"]), gy, chunk_len=chunk,
                                     times=t, layout="array")
    dxs, dzs, dls = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk)
    torch.cuda.synchronize()
    # inputs in (two logits, two lambdas), gradients out (the same four)
    assert t.as_dict()["layout"]["launches"] == 8
    dza, dla = _scan(dza), _scan(dla)
    assert torch.equal(dxa, dxs)
    for d in range(4):
        assert torch.equal(dla[d], dls[d])
        if shared:  # fp32 atomic channel sums: equal up to their order
            assert torch.allclose(dza[d].float(), dzs[d].float(), rtol=2e-2, atol=1e-2)
        else:
            assert torch.equal(dza[d], dzs[d])
    rdx, rdl, rdz = oracle.backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk=chunk)
    errs = {"dx": oracle.normwise_error(_np(dxa), rdx)}
    for d in range(4):
        errs["dlam%d" % d] = oracle.normwise_error(_np(dla[d]), rdl[d])
        errs["dlogits%d" % d] = oracle.normwise_error(_np(dza[d]), rdz[d])
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("name,planes", [
    ("profile", [(0, 0), (15, 7)]),
    ("wide", [(0, 0), (0, 1151)]),
])
def test_full_size_array_layout_sampled_planes(name, planes):
    """The bench's full-size workloads in the array layout, checked on
    sampled planes that the oracle computes on their own."""
    wl = WORKLOADS[name]
    _say("full %s, array layout" % name)
    inp = make_inputs(wl, DEV)
    za, la = _array(inp["logits"]), _array(inp["lam"])
    del inp["logits"], inp["lam"]
    got = G.gspn_forward4(inp["x"], za, la, workspace=G.forward4_workspace(inp["x"], wl.cw, "array"),
                          layout="array")
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    for n, c in planes:
        wc = 0 if wl.shared_w else c
        # the plane's per-direction tensors, back in their scan frames for the oracle
        zs = _scan([z[n:n + 1, wc:wc + 1] for z in za])
        ls = _scan([l[n:n + 1, c:c + 1] for l in la])
        ref = oracle.forward4(_np(inp["x"][n:n + 1, c:c + 1]), [_np(z) for z in zs], [_np(l) for l in ls])
        e = oracle.normwise_error(_np(got[n:n + 1, c:c + 1]), ref)
        _say("  plane (%d, %d): normwise error %.3g" % (n, c, e))
        assert e <= TOL[wl.dtype]
