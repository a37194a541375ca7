"""GPU parity of the compressive-proxy backward: gspn_proxy_backward4 (through
the C ABI) against the fp64 oracle's chain-rule gradient on the same seeded
inputs and dL/dy.  Tolerances, normwise per output tensor: 1e-5 for fp32
storage; 2e-2 for bf16 storage, whose four proxy-space intermediates (x_p,
y_p, dL/dy_p, dx_p) each round once to bf16 on top of the propagation's own
bf16 rounding.  The cases cover the matrix-core path with the projection
folded in (c <= 320, pixel counts in multiples of 128), the one with channel
groups and the projection apart (c > 320), the VALU sums (ragged pixel
counts, fp32), both logit sharings, chunks and learnable merges."""
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


def _gy(wl, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    t = torch.randn((wl.n, wl.c, wl.h, wl.w), generator=g, device=DEV, dtype=torch.float32)
    return t.to(wl.torch_dtype)


def _merge(cp, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.randn((4, cp), generator=g, device=DEV, dtype=torch.float32)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield
    torch.cuda.synchronize()


def _errors(got, ref):
    names = ["dx", "dw_down", "dw_up"]
    errs = {k: oracle.normwise_error(_np(got[i]), ref[i]) for i, k in enumerate(names)}
    for d in range(4):
        errs["dlogits%d" % d] = oracle.normwise_error(_np(got[3][d]), ref[4][d])
        errs["dlam%d" % d] = oracle.normwise_error(_np(got[4][d]), ref[3][d])
    if len(got) > 5:
        errs["dmerge"] = oracle.normwise_error(_np(got[5]), ref[5])
    return errs


@pytest.mark.parametrize("shape,dtype,shared,chunk,merge", [
    ((1, 40, 32, 64, 8), "bf16", True, 0, False),      # folded projection, two channel blocks
    ((2, 320, 32, 128, 8), "bf16", True, 0, True),     # folded, ten channel blocks, two images
    ((1, 96, 48, 256, 16), "bf16", False, 7, False),   # sixteen proxy channels, chunks
    ((1, 336, 16, 128, 6), "bf16", True, 0, False),    # two channel groups, projection apart
    ((2, 64, 33, 47, 4), "bf16", True, 5, True),       # ragged pixel count: VALU sums
    ((1, 24, 20, 30, 3), "f32", False, 0, False),      # plane-resident proxy-space backward
    ((2, 40, 72, 40, 5), "f32", True, 9, True),        # fp32, shared logits, chunks, merge
    ((1, 20, 16, 128, 4), "bf16", True, 0, False),     # channels not a multiple of 8: VALU sums
    ((1, 48, 24, 64, 24), "bf16", False, 0, False),    # more than 16 proxy channels: VALU sums
])
def test_proxy_backward_small(shape, dtype, shared, chunk, merge):
    n, c, h, w, cp = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 31 + h + c, c_proxy=cp)
    _say("proxy backward %s %s shared=%s chunk=%d merge=%s" % (shape, dtype, shared, chunk, merge))
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 101 + w)
    m = _merge(cp, 7) if merge else None
    got = G.gspn_proxy_backward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], gy,
                                 chunk_len=chunk, merge=m)
    torch.cuda.synchronize()
    ref = oracle.proxy_backward4(_np(inp["x"]), _np(inp["w_down"]), _np(inp["w_up"]),
                                 [_np(z) for z in inp["logits"]], [_np(l) for l in inp["lam"]], _np(gy),
                                 chunk=chunk, merge=None if m is None else _np(m))
    errs = _errors(got, ref)
    _say("  worst normwise error %.3g (%s)" % (max(errs.values()), max(errs, key=errs.get)))
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_proxy_backward_array_layout(dtype):
    """The per-direction logits and lambdas in the array frame ([.., H, W]
    for every direction): the same gradients as the scan layout, the
    horizontal ones returned in the array frame."""
    wl = Workload("case", 1, 64, 40, 128, dtype, True, 0, 55, c_proxy=8)
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 9)
    za = [z if d < 2 else z.transpose(-1, -2).contiguous() for d, z in enumerate(inp["logits"])]
    la = [l if d < 2 else l.transpose(-1, -2).contiguous() for d, l in enumerate(inp["lam"])]
    a = G.gspn_proxy_backward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], gy)
    b = G.gspn_proxy_backward4(inp["x"], inp["w_down"], inp["w_up"], za, la, gy, layout="array")
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.allclose(a[i].float(), b[i].float(), rtol=1e-5, atol=1e-6), i
    for d in range(4):
        back = (lambda t: t) if d < 2 else (lambda t: t.transpose(-1, -2))
        assert torch.equal(a[4][d], back(b[4][d]))
        # shared-logit sums are fp32 atomics: equal up to their order
        assert torch.allclose(a[3][d].float(), back(b[3][d]).float(), rtol=2e-2, atol=1e-3)


def test_proxy_backward_timed_stages():
    """The timed variant gives the same gradients and reports the stages the
    header names: x's projection, dx's projection, the two passes summing the
    weight gradients' partials (over gy with dL/dy_p's projection folded in,
    and over x), and the proxy-space forward and adjoint."""
    wl = Workload("case", 1, 64, 32, 128, "bf16", True, 0, 77, c_proxy=8)
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 5)
    a = G.gspn_proxy_backward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], gy)
    t = G.StageTimes()
    b = G.gspn_proxy_backward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], gy, times=t)
    torch.cuda.synchronize()
    st = t.as_dict()
    _say("  stages: %s" % {k: v for k, v in st.items() if isinstance(v, dict) and v.get("launches")})
    assert st["project_down"]["launches"] == 1 and st["project_up"]["launches"] == 1
    assert st["weight_grad"]["launches"] == 2
    assert st["reduce"]["launches"] >= 4            # two weight transposes, two reductions
    assert st["adjoint"]["launches"] >= 1 and st["scan"]["launches"] >= 1
    for i in range(3):
        assert torch.equal(a[i], b[i]), i
    for d in range(4):
        assert torch.equal(a[4][d], b[4][d])


@pytest.mark.parametrize("shape", [(1, 80, 16, 128, 8), (1, 40, 21, 37, 3)])
def test_proxy_backward_deterministic(shape):
    """Per-channel logits and no merge: every output, the weight gradients
    among them, is the same bit for bit on a second call."""
    n, c, h, w, cp = shape
    wl = Workload("case", n, c, h, w, "bf16", False, 0, 9, c_proxy=cp)
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 6)
    a = G.gspn_proxy_backward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], gy)
    b = G.gspn_proxy_backward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], gy)
    torch.cuda.synchronize()
    for i in range(3):
        assert torch.equal(a[i], b[i]), i
    for j in (3, 4):
        for d in range(4):
            assert torch.equal(a[j][d], b[j][d]), (j, d)


def test_proxy_backward_no_pixels():
    """n = 0: the weight gradients and dmerge are sums over no pixels, written
    as zeros."""
    c, cp, h, w = 16, 4, 8, 8
    x = torch.empty((0, c, h, w), device=DEV, dtype=torch.bfloat16)
    wd = torch.randn((cp, c), device=DEV).to(torch.bfloat16)
    wu = torch.randn((c, cp), device=DEV).to(torch.bfloat16)
    zs = [torch.empty((0, 1, 3) + G.frame_shape(d, h, w), device=DEV, dtype=torch.bfloat16) for d in range(4)]
    ls = [torch.empty((0, cp) + G.frame_shape(d, h, w), device=DEV, dtype=torch.bfloat16) for d in range(4)]
    dm = torch.full((4, cp), 7.0, device=DEV)
    res = G.gspn_proxy_backward4(x, wd, wu, zs, ls, torch.empty_like(x), merge=torch.ones((4, cp), device=DEV),
                                 dmerge=dm)
    torch.cuda.synchronize()
    assert res[0].numel() == 0
    assert torch.all(res[1] == 0) and torch.all(res[2] == 0) and torch.all(res[5] == 0)


def test_proxy4_autograd():
    """gspn_proxy4 under autograd gives gspn_proxy_backward4's gradients
    (weight gradients cast to the weights' dtype)."""
    wl = Workload("case", 1, 32, 16, 128, "f32", True, 0, 12, c_proxy=4)
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 8)
    m = _merge(4, 3)
    leaves = [inp["x"], inp["w_down"], inp["w_up"], m] + list(inp["logits"]) + list(inp["lam"])
    for t in leaves:
        t.requires_grad_(True)
    y = G.gspn_proxy4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], merge=m)
    y.backward(gy)
    ref = G.gspn_proxy_backward4(inp["x"].detach(), inp["w_down"].detach(), inp["w_up"].detach(),
                                 [z.detach() for z in inp["logits"]], [l.detach() for l in inp["lam"]], gy,
                                 merge=m.detach())
    torch.cuda.synchronize()
    assert torch.equal(inp["x"].grad, ref[0])
    assert torch.allclose(inp["w_down"].grad, ref[1], rtol=1e-6, atol=1e-6)
    assert torch.allclose(inp["w_up"].grad, ref[2], rtol=1e-6, atol=1e-6)
    assert torch.allclose(m.grad, ref[5], rtol=1e-5, atol=1e-5)
    for d in range(4):
        assert torch.allclose(inp["logits"][d].grad, ref[3][d], rtol=1e-5, atol=1e-6)
        assert torch.equal(inp["lam"][d].grad, ref[4][d])


def test_full_size_proxy_backward():
    """The 2048^2, N = 1, C = 320 -> C_proxy = 8 bf16 workload with
    channel-shared logits, in the launch configuration the bench times.  The
    oracle runs the whole proxy space (eight 2048^2 planes, fp64): every
    proxy-space gradient and both weight gradients are compared whole, dx on
    three sampled channels."""
    wl = WORKLOADS["proxy"]
    _say("full proxy backward")
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 404)
    got = G.gspn_proxy_backward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], gy,
                                 workspace=G.proxy_backward4_workspace(inp["x"], wl.c_proxy, wl.cw))
    torch.cuda.synchronize()
    dx, dwd, dwu, dz, dl = got
    assert torch.isfinite(dx).all() and torch.isfinite(dwd).all() and torch.isfinite(dwu).all()
    wd = _np(inp["w_down"])
    wu = _np(inp["w_up"])
    zs = [_np(z) for z in inp["logits"]]
    ls = [_np(l) for l in inp["lam"]]
    x = _np(inp["x"])
    xp = oracle.project(x, wd)
    yp = oracle.forward4(xp, zs, ls)
    g = _np(gy)
    gp = oracle.project(g, wu.T)
    rdwu = g[0].reshape(wl.c, -1) @ yp[0].reshape(wl.c_proxy, -1).T
    del g, yp
    _say("  dw_up normwise error %.3g" % oracle.normwise_error(_np(dwu), rdwu))
    assert oracle.normwise_error(_np(dwu), rdwu) <= TOL["bf16"]
    rdxp, rdl, rdz = oracle.backward4(xp, zs, ls, gp)
    del gp, xp
    for d in range(4):
        el = oracle.normwise_error(_np(dl[d]), rdl[d])
        ez = oracle.normwise_error(_np(dz[d]), rdz[d])
        _say("  direction %d: dlam %.3g, dlogits %.3g" % (d, el, ez))
        assert el <= TOL["bf16"] and ez <= TOL["bf16"]
    rdwd = rdxp[0].reshape(wl.c_proxy, -1) @ x[0].reshape(wl.c, -1).T
    del x
    _say("  dw_down normwise error %.3g" % oracle.normwise_error(_np(dwd), rdwd))
    assert oracle.normwise_error(_np(dwd), rdwd) <= TOL["bf16"]
    chans = [0, 161, 319]
    rdx = oracle.project(rdxp, wd.T[chans])
    for j, c in enumerate(chans):
        e = oracle.normwise_error(_np(dx[:, c:c + 1]), rdx[:, j:j + 1])
        _say("  dx channel %d: normwise error %.3g" % (c, e))
        assert e <= TOL["bf16"]


@pytest.mark.parametrize("shape,dtype,shared,chunk,merge", [
    ((1, 40, 96, 128, 8), "bf16", True, 0, True),     # planes above 64 x 64: the fp32 scans kept too
    ((2, 64, 64, 200, 4), "bf16", False, 9, False),   # per-channel logits, chunks
    ((1, 24, 40, 48, 3), "f32", True, 0, False),      # planes of at most 64 x 64: x_p and y_p only
])
def test_proxy_backward_from_kept_states(shape, dtype, shared, chunk, merge):
    """gspn_proxy_forward4 keeping its proxy-space state (x_p, y_p, the fp32
    scans), then gspn_proxy_backward4 reading it: the forward agrees with the
    oracle, and the gradients are those of the recomputing backward (bit for
    bit, but the fp32-atomic sums of shared logits and of dmerge, up to their
    order), so also the oracle's."""
    n, c, h, w, cp = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 77 + h + c, c_proxy=cp)
    _say("proxy backward from kept states %s %s shared=%s chunk=%d merge=%s" % (shape, dtype, shared, chunk, merge))
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 201 + w)
    m = _merge(cp, 8) if merge else None
    args = (inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"])
    y, st = G.gspn_proxy_forward4(*args, chunk_len=chunk, merge=m, states=True)
    kept = G.gspn_proxy_backward4(*args, gy, chunk_len=chunk, merge=m, states=st)
    full = G.gspn_proxy_backward4(*args, gy, chunk_len=chunk, merge=m)
    torch.cuda.synchronize()
    ref_y = oracle.proxy_forward4(_np(inp["x"]), _np(inp["w_down"]), _np(inp["w_up"]),
                                  [_np(z) for z in inp["logits"]], [_np(l) for l in inp["lam"]], chunk=chunk,
                                  merge=None if m is None else _np(m))
    assert oracle.normwise_error(_np(y), ref_y) <= TOL[dtype]
    for i in range(3):   # dx, dw_down, dw_up
        assert torch.equal(kept[i], full[i]), i
    for d in range(4):
        assert torch.equal(kept[4][d], full[4][d]), d   # dlambda
        if shared:
            assert oracle.normwise_error(_np(kept[3][d]), _np(full[3][d])) <= 1e-2, d
        else:
            assert torch.equal(kept[3][d], full[3][d]), d
    if merge:
        assert oracle.normwise_error(_np(kept[5]), _np(full[5])) <= 1e-5
    ref = oracle.proxy_backward4(_np(inp["x"]), _np(inp["w_down"]), _np(inp["w_up"]),
                                 [_np(z) for z in inp["logits"]], [_np(l) for l in inp["lam"]], _np(gy),
                                 chunk=chunk, merge=None if m is None else _np(m))
    errs = _errors(kept, ref)
    _say("  worst normwise error %.3g (%s)" % (max(errs.values()), max(errs, key=errs.get)))
    assert max(errs.values()) <= TOL[dtype], errs


def test_proxy_autograd_keeping_states():
    """gspn_proxy4(keep_states=True) as a training step: the same gradients
    as without kept states."""
    wl = Workload("case", 1, 32, 96, 128, "bf16", True, 0, 91, c_proxy=8)
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 17)
    grads = []
    for keep in (False, True):
        x = inp["x"].clone().requires_grad_(True)
        wd = inp["w_down"].clone().requires_grad_(True)
        wu = inp["w_up"].clone().requires_grad_(True)
        lams = [l.clone().requires_grad_(True) for l in inp["lam"]]
        y = G.gspn_proxy4(x, wd, wu, inp["logits"], lams, keep_states=keep)
        y.backward(gy)
        grads.append([x.grad, wd.grad, wu.grad] + [l.grad for l in lams])
    torch.cuda.synchronize()
    for a, b in zip(*grads):
        assert torch.equal(a, b)
