"""GPU tests of the forward that keeps its states for the backward:
gspn_forward4 with ``states`` (through the C ABI) writes the four directions'
unweighted scans in fp32, each in its scan frame, which match the fp64
oracle's single-direction scans; y is unchanged; and gspn_backward4 given
those states returns the gradients of the recomputing backward bit for bit
(the same kernel computes the states both ways).  Tolerances as in the
parity tests: 1e-5 normwise for fp32 storage, 2e-2 for bf16."""
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


CASES = [
    # (dtype, (n, c, h, w), shared, chunk)
    ("f32", (2, 3, 70, 90), False, 0),     # the four-direction launch either way
    ("f32", (2, 3, 70, 90), False, 9),
    ("bf16", (1, 4, 100, 130), True, 0),   # shared weights as half pairs
    ("bf16", (2, 2, 72, 40), False, 7),
    # very few long lines: the banded forward writes the states, the banded
    # adjoint reads them (unchunked) or the one-line adjoint does (chunked)
    ("f32", (1, 3, 512, 600), False, 0),
    ("bf16", (1, 2, 520, 512), True, 0),
    ("bf16", (2, 2, 512, 544), False, 100),
]


@pytest.mark.parametrize("merge", [False, True])
@pytest.mark.parametrize("dtype,shape,shared,chunk", CASES)
def test_forward_states(dtype, shape, shared, chunk, merge):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 301 + h + w)
    _say("forward states %s %s shared=%s chunk=%d merge=%s" % (shape, dtype, shared, chunk, merge))
    inp = make_inputs(wl, DEV)
    m = torch.randn((4, c), device=DEV) if merge else None
    ws = G.forward4_workspace(inp["x"], wl.cw)
    y, st = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk, workspace=ws, merge=m,
                            states=True)
    plain = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk, workspace=ws, merge=m)
    torch.cuda.synchronize()
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk, merge=None if m is None else _np(m))
    assert oracle.normwise_error(_np(y), ref) <= TOL[dtype]
    if dtype == "f32" and h > 64:
        # same maps, same merge: the same y
        assert torch.equal(y, plain)
    else:
        assert oracle.normwise_error(_np(plain), ref) <= TOL[dtype]
    for d in range(4):
        got = _np(G.state_map(st, d, shape))
        want = oracle.scan(d, inp["x"], inp["logits"][d], inp["lam"][d], chunk)
        if d >= 2:
            want = want.transpose(0, 1, 3, 2)  # the horizontal directions' scan frame
        err = oracle.normwise_error(got, want)
        assert err <= TOL[dtype], (d, err)


@pytest.mark.parametrize("merge", [False, True])
@pytest.mark.parametrize("dtype,shape,shared,chunk", CASES)
def test_backward_from_states(dtype, shape, shared, chunk, merge):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 401 + h + w)
    _say("backward from states %s %s shared=%s chunk=%d merge=%s" % (shape, dtype, shared, chunk, merge))
    inp = make_inputs(wl, DEV)
    m = torch.randn((4, c), device=DEV) if merge else None
    g = torch.Generator(device=DEV)
    g.manual_seed(wl.seed + 7)
    gy = torch.randn((n, c, h, w), generator=g, device=DEV, dtype=torch.float32).to(wl.torch_dtype)
    _, st = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk,
                            workspace=G.forward4_workspace(inp["x"], wl.cw), merge=m, states=True)
    a = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk, merge=m, dmerge=True,
                         states=st)
    b = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk, merge=m, dmerge=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])
    for d in range(4):
        assert torch.equal(a[2][d], b[2][d])
        if shared:   # sums over channels in fp32 atomics, whose order varies
            assert torch.allclose(a[1][d].float(), b[1][d].float(), rtol=1e-5, atol=1e-6)
        else:
            assert torch.equal(a[1][d], b[1][d])
    # dmerge: fp32 atomic sums in an order that varies between calls, each
    # entry a sum with cancellation, so compared normwise
    assert (a[3] - b[3]).abs().max() <= 1e-5 * b[3].abs().max()
    o = oracle.backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk=chunk, merge=None if m is None else _np(m))
    assert oracle.normwise_error(_np(a[0]), o[0]) <= TOL[dtype]
    for d in range(4):
        assert oracle.normwise_error(_np(a[2][d]), o[1][d]) <= TOL[dtype]
        assert oracle.normwise_error(_np(a[1][d]), o[2][d]) <= TOL[dtype]


SMALL = [
    # planes of at most 64 x 64 leave their one-pass path when the states are kept
    ("f32", (2, 3, 23, 41), False, 5),     # ragged lines: lanes past the end of every line
    ("bf16", (1, 5, 40, 72), True, 0),     # channel groups of three in the adjoint, the last ragged
    ("f32", (1, 2, 64, 64), False, 7),
]


@pytest.mark.parametrize("dtype,shape,shared,chunk", SMALL)
def test_kept_states_on_small_planes(dtype, shape, shared, chunk):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 501 + h + w)
    _say("kept states, small planes %s %s shared=%s chunk=%d" % (shape, dtype, shared, chunk))
    inp = make_inputs(wl, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(wl.seed + 3)
    gy = torch.randn((n, c, h, w), generator=g, device=DEV, dtype=torch.float32).to(wl.torch_dtype)
    y, st = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk,
                            workspace=G.forward4_workspace(inp["x"], wl.cw), states=True)
    dx, dz, dl = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk, states=st)
    torch.cuda.synchronize()
    assert oracle.normwise_error(_np(y), oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk)) \
        <= TOL[dtype]
    o = oracle.backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk=chunk)
    assert oracle.normwise_error(_np(dx), o[0]) <= TOL[dtype]
    for d in range(4):
        assert oracle.normwise_error(_np(dl[d]), o[1][d]) <= TOL[dtype]
        assert oracle.normwise_error(_np(dz[d]), o[2][d]) <= TOL[dtype]


def test_tstage_training_step_keeping_states():
    """The 64 x 96 x 56 x 56 stage map, fp32: forward keeping its states, then
    the backward from them with the binding's smaller workspace.  Lanes past
    the end of a 56-position line once read their left neighbour's state
    past the end of the states buffer here; the gradients are checked on
    sampled planes that the oracle computes on their own."""
    wl = WORKLOADS["tstage"]
    _say("tstage training step keeping states")
    inp = make_inputs(wl, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(41)
    gy = torch.randn((wl.n, wl.c, wl.h, wl.w), generator=g, device=DEV, dtype=torch.float32)
    y, st = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], workspace=G.forward4_workspace(inp["x"], wl.cw),
                            states=True)
    t = G.StageTimes()
    dx, dz, dl = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, states=st, times=t)
    torch.cuda.synchronize()
    stages = t.as_dict()
    assert stages["scan"]["launches"] == 0 and stages["adjoint"]["launches"] == 1
    assert torch.isfinite(dx).all() and torch.isfinite(y).all()
    for pn, pc in [(0, 0), (63, 95), (17, 40)]:
        sl = (slice(pn, pn + 1), slice(pc, pc + 1))
        zs = [z[sl] for z in inp["logits"]]
        ls = [l[sl] for l in inp["lam"]]
        assert oracle.normwise_error(_np(y[sl]), oracle.forward4(inp["x"][sl], zs, ls)) <= TOL["f32"]
        o = oracle.backward4(inp["x"][sl], zs, ls, gy[sl])
        errs = [oracle.normwise_error(_np(dx[sl]), o[0])]
        for d in range(4):
            errs += [oracle.normwise_error(_np(dl[d][sl]), o[1][d]), oracle.normwise_error(_np(dz[d][sl]), o[2][d])]
        _say("  plane (%d, %d): worst normwise error %.3g" % (pn, pc, max(errs)))
        assert max(errs) <= TOL["f32"]


def test_backward_from_states_takes_the_smaller_workspace():
    wl = Workload("case", 1, 2, 80, 96, "f32", False, 0, 77)
    inp = make_inputs(wl, DEV)
    _, st = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], workspace=G.forward4_workspace(inp["x"], 2),
                            states=True)
    gy = torch.randn_like(inp["x"])
    full = G.backward4_workspace(inp["x"], 2)
    small = G.backward4_workspace(inp["x"], 2, with_states=True)
    assert small.numel() == full.numel() - 16 * inp["x"].numel()
    t = G.StageTimes()
    a = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, workspace=small, states=st, times=t)
    b = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, workspace=full)
    torch.cuda.synchronize()
    stages = t.as_dict()
    assert stages["scan"]["launches"] == 0          # no recompute
    assert torch.equal(a[0], b[0])
    for d in range(4):
        assert torch.equal(a[1][d], b[1][d]) and torch.equal(a[2][d], b[2][d])


@pytest.mark.parametrize("keep", [False, True])
def test_gspn4_keeps_states(keep):
    wl = Workload("case", 2, 3, 70, 80, "f32", False, 0, 55)
    inp = make_inputs(wl, DEV)
    x = inp["x"].clone().requires_grad_(True)
    zs = [z.clone().requires_grad_(True) for z in inp["logits"]]
    ls = [l.clone().requires_grad_(True) for l in inp["lam"]]
    y = G.gspn4(x, zs, ls, keep_states=keep)
    gy = torch.randn_like(y)
    grads = torch.autograd.grad(y, [x] + zs + ls, gy)
    ref = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy)
    torch.cuda.synchronize()
    assert torch.equal(grads[0], ref[0])
    for d in range(4):
        assert torch.equal(grads[1 + d], ref[1][d]) and torch.equal(grads[5 + d], ref[2][d])
