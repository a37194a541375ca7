"""GPU parity: libgspn (through its C ABI) against the fp64 CPU oracle on the
same seeded inputs.

Tolerances (normwise, max|gpu - oracle| / max|oracle| per output): 1e-5 for
fp32 storage, 2e-2 for bf16 storage with fp32 arithmetic.  Small cases
compare every element; the full-size workloads run exactly the call the
bench times and compare sampled planes that the oracle computes on its own.
"""
import math
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


def _err(got, ref):
    return oracle.normwise_error(_np(got), ref)


def _wl(name="case", n=1, c=2, h=16, w=16, dtype="f32", shared=False, chunk=0, seed=11, cp=0):
    return Workload(name, n, c, h, w, dtype, shared, chunk, seed, c_proxy=cp)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield
    torch.cuda.synchronize()


# ----------------------------------------------------------------------------
# Small cases: every element
# ----------------------------------------------------------------------------

SMALL_SHAPES = [
    (1, 2, 16, 16),      # the tiny workload
    (2, 3, 37, 70),      # ragged, one wave per line
    (1, 2, 70, 37),
    (1, 2, 9, 300),      # P = 2, three waves per vertical line
    (1, 1, 300, 9),
    (1, 2, 5, 1000),     # P = 4, four waves
    (1, 1, 3, 3000),     # P = 8 with 384 lanes (long-line variant)
    (1, 1, 3000, 3),
    (1, 3, 1, 17),       # single-line scans
    (1, 3, 17, 1),       # line length 1
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SMALL_SHAPES)
@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_scan_each_direction(direction, shape, dtype):
    n, c, h, w = shape
    wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, seed=100 + h + w)
    _say("scan dir=%d shape=%s %s" % (direction, shape, dtype))
    inp = make_inputs(wl, DEV)
    got = G.gspn_scan_fwd(direction, inp["x"], inp["logits"][direction], inp["lam"][direction])
    torch.cuda.synchronize()
    ref = oracle.scan(direction, inp["x"], inp["logits"][direction], inp["lam"][direction])
    assert _err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("chunk", [1, 3, 8, 16, 40])
@pytest.mark.parametrize("direction", [0, 1, 2, 3])
def test_scan_chunked(direction, chunk):
    wl = _wl(n=2, c=2, h=37, w=29, seed=7)
    _say("chunked dir=%d chunk=%d" % (direction, chunk))
    inp = make_inputs(wl, DEV)
    got = G.gspn_scan_fwd(direction, inp["x"], inp["logits"][direction], inp["lam"][direction],
                          chunk_len=chunk)
    torch.cuda.synchronize()
    ref = oracle.scan(direction, inp["x"], inp["logits"][direction], inp["lam"][direction],
                      chunk=chunk)
    assert _err(got, ref) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_scan_shared_weights_and_accumulate(dtype):
    wl = _wl(n=2, c=5, h=33, w=40, dtype=dtype, shared=True, seed=5)
    _say("shared+accumulate %s" % dtype)
    inp = make_inputs(wl, DEV)
    base = torch.randn(inp["x"].shape, device=DEV).to(inp["x"].dtype)
    for d in range(4):
        out = base.clone()
        G.gspn_scan_fwd(d, inp["x"], inp["logits"][d], inp["lam"][d], out=out, accumulate=True)
        torch.cuda.synchronize()
        ref = _np(base) + oracle.scan(d, inp["x"], inp["logits"][d], inp["lam"][d])
        assert _err(out, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_normalize_and_prenormalised_scan(dtype):
    wl = _wl(n=1, c=3, h=20, w=45, dtype=dtype, seed=9)
    _say("normalize %s" % dtype)
    inp = make_inputs(wl, DEV)
    for d in range(4):
        w = G.gspn_normalize_weights(d, inp["logits"][d], wl.h, wl.w)
        torch.cuda.synchronize()
        ref = oracle.normalize(d, inp["logits"][d])
        tol = 1e-6 if dtype == "f32" else 8e-3
        assert np.max(np.abs(_np(w) - ref)) <= tol
        # scan with the stored weights equals the oracle given those weights
        got = G.gspn_scan_fwd(d, inp["x"], w, inp["lam"][d], wts_are_logits=False)
        torch.cuda.synchronize()
        ref_h = oracle.scan(d, inp["x"], w, inp["lam"][d], wts_are_logits=False)
        assert _err(got, ref_h) <= TOL[dtype]


def _ulps(got, ref):
    """|got - ref| in units in the last place of fp32 at ref (normal range)."""
    ref = np.asarray(ref, dtype=np.float64)
    ulp = np.ldexp(1.0, np.floor(np.log2(np.abs(ref))).astype(np.int64) - 23)
    return np.abs(np.asarray(got, dtype=np.float64) - ref) / ulp


def test_sigmoid_weights_ulps():
    """The sigmoid (the standard logistic, evaluated to about 2 ulp) through
    the normalisation kernel.  Lines of two positions: each position has one
    missing neighbour, its centre logit is 20 and its other neighbour's logit
    z sweeps [-20, 20], so its side weight is s(z) / (s(z) + s(20)); for z <= 0
    that is s(z) to within a factor near 1, and its error is the sigmoid's plus
    the normalisation's (a sum, a refined reciprocal and a product: under 2
    ulp).  Bound: 4 ulp."""
    S = 65536
    z = np.linspace(-20.0, 20.0, S, dtype=np.float32)
    logits = np.zeros((1, 1, 3, S, 2), dtype=np.float32)
    logits[0, 0, 1] = 20.0
    logits[0, 0, 2, :, 0] = z      # position 0: neighbour k+1
    logits[0, 0, 0, :, 1] = z      # position 1: neighbour k-1
    t = torch.from_numpy(logits).to(DEV)
    w = _np(G.gspn_normalize_weights(0, t, S, 2))
    torch.cuda.synchronize()
    ref = oracle.normalize(0, logits)
    side = np.concatenate([w[0, 0, 2, :, 0], w[0, 0, 0, :, 1]])
    side_ref = np.concatenate([ref[0, 0, 2, :, 0], ref[0, 0, 0, :, 1]])
    u = _ulps(side, side_ref)
    _say("sigmoid side weights: max %.2f ulp, mean %.3f ulp" % (u.max(), u.mean()))
    assert u.max() <= 4.0
    centre = np.concatenate([w[0, 0, 1, :, 0], w[0, 0, 1, :, 1]])
    assert _ulps(centre, np.concatenate([ref[0, 0, 1, :, 0], ref[0, 0, 1, :, 1]])).max() <= 4.0


def test_normalize_extreme_logit_rows():
    """Rows whose every existing logit lies below about -69: there each
    sigmoid is about e^z and an fp32 row sum could underflow to 0 (0/0 =
    NaN); the kernels must still give the oracle's finite normalised row,
    in the standalone normalisation and inside the scans."""
    wl = _wl(n=1, c=2, h=24, w=40, seed=61)
    inp = make_inputs(wl, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    zs = [(-120.0 + 50.0 * torch.rand(z.shape, generator=g, device=DEV)).contiguous() for z in inp["logits"]]
    for d in range(4):
        w = G.gspn_normalize_weights(d, zs[d], wl.h, wl.w)
        torch.cuda.synchronize()
        assert torch.isfinite(w).all()
        ref = oracle.normalize(d, zs[d])
        assert np.max(np.abs(_np(w) - ref)) <= 1e-6
    y = G.gspn_forward4(inp["x"], zs, inp["lam"], workspace=G.forward4_workspace(inp["x"], wl.cw))
    y0 = G.gspn_forward4(inp["x"], zs, inp["lam"])
    torch.cuda.synchronize()
    ref = oracle.forward4(inp["x"], zs, inp["lam"])
    assert _err(y, ref) <= TOL["f32"] and _err(y0, ref) <= TOL["f32"]


def test_merge4():
    hs = [torch.randn(3, 5, 17, 19, device=DEV) for _ in range(4)]
    y = G.gspn_merge4(hs)
    torch.cuda.synchronize()
    ref = sum(_np(h) for h in hs)
    assert np.max(np.abs(_np(y) - ref)) <= 1e-5


@pytest.mark.parametrize("hw", [(13, 29), (16, 32), (8, 24)])   # ragged (VALU) / 128 or 64 pixels per wave (MFMA, bf16)
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("cin,cout", [(320, 8), (8, 320), (37, 5), (3, 11), (40, 16), (64, 17), (5, 33), (520, 8)])
def test_project(cin, cout, dtype, hw):
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    g = torch.Generator(device=DEV).manual_seed(cin * 1000 + cout)
    x = torch.randn(2, cin, hw[0], hw[1], device=DEV, generator=g).to(tdt)
    wt = (torch.randn(cout, cin, device=DEV, generator=g) / math.sqrt(cin)).to(tdt)
    _say("project %d->%d %s" % (cin, cout, dtype))
    got = G.gspn_proxy_project(x, wt)
    torch.cuda.synchronize()
    ref = oracle.project(x, wt)
    assert _err(got, ref) <= (1e-5 if dtype == "f32" else 1e-2)


@pytest.mark.parametrize("use_ws", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [0, 8, 5])
@pytest.mark.parametrize("shape", [(1, 2, 16, 16), (2, 3, 23, 41), (1, 2, 64, 64), (2, 2, 65, 33), (1, 2, 40, 72),
                                   (1, 2, 64, 130), (1, 1, 1100, 40),
                                   (1, 3, 1, 17), (2, 2, 17, 1), (1, 2, 1, 1)])   # single rows, columns, positions
def test_forward4_small(shape, chunk, dtype, use_ws):
    n, c, h, w = shape
    for shared in (False, True):
        wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, shared=shared, seed=h * w + chunk)
        _say("forward4 %s chunk=%d %s shared=%s ws=%s" % (shape, chunk, dtype, shared, use_ws))
        inp = make_inputs(wl, DEV)
        ws = G.forward4_workspace(inp["x"], wl.cw) if use_ws else None
        got = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk, workspace=ws)
        torch.cuda.synchronize()
        ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk)
        assert _err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,chunk", [((1, 2, 16, 16), 0), ((2, 3, 23, 41), 0), ((2, 3, 23, 41), 7),
                                         ((1, 2, 1030, 70), 0), ((1, 1, 70, 1500), 9),
                                         ((1, 2, 2048, 33), 0)])
def test_scan4_outputs(shape, chunk, dtype):
    n, c, h, w = shape
    wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, seed=h + 3 * w + chunk)
    _say("scan4 %s chunk=%d %s" % (shape, chunk, dtype))
    inp = make_inputs(wl, DEV)
    outs = G.gspn_scan4_fwd(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk)
    torch.cuda.synchronize()
    for d in range(4):
        ref = oracle.scan(d, inp["x"], inp["logits"][d], inp["lam"][d], chunk=chunk)
        assert _err(outs[d], ref) <= TOL[dtype], d


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [0, 7])
@pytest.mark.parametrize("shape", [
    (1, 3, 40, 72),     # long-line kernel
    (2, 4, 40, 70),     # one workgroup per line (70 is not a whole number of vectors)
    (1, 2, 30, 2100),   # lines longer than the fused launch takes: one launch per direction
    (2, 3, 50, 60),     # plane-resident kernel (logits normalised per channel)
])
def test_forward4_shared_weights(shape, chunk, dtype):
    """Channel-shared logits over several channels: normalised once per
    direction into fp32 triples (fp32 storage) or packed half pairs (bf16)."""
    n, c, h, w = shape
    wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, shared=True, chunk=chunk, seed=41 + w)
    _say("forward4 shared %s chunk=%d %s" % (shape, chunk, dtype))
    inp = make_inputs(wl, DEV)
    got = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk,
                          workspace=G.forward4_workspace(inp["x"], wl.cw))
    torch.cuda.synchronize()
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk)
    assert _err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("chunk", [0, 5])
@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("dtype,shape", [
    ("bf16", (1, 2, 24, 560)),   # 70 lanes of 8 positions: a second wave with 6 lanes on the line
    ("f32", (1, 2, 36, 280)),    # 70 lanes of 4 positions
    ("bf16", (2, 1, 16, 1032)),  # 129 lanes: a third wave with one lane on the line
])
def test_long_line_kernel_partial_waves(dtype, shape, shared, chunk):
    """The long-line kernel with lines that end inside a wave after the first:
    the lanes past the line must not leak into it."""
    n, c, h, w = shape
    wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, shared=shared, chunk=chunk, seed=61 + w)
    _say("long-line partial waves %s %s shared=%s chunk=%d" % (shape, dtype, shared, chunk))
    inp = make_inputs(wl, DEV)
    got, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk,
                                       workspace=G.forward4_workspace(inp["x"], wl.cw))
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "scan4lp_kernel", times["scan_kernel"]
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk)
    assert _err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", [
    (1, 1031, 8, 72),   # an odd plane count: the last workgroup has a plane too few
    (2, 515, 8, 72),    # a workgroup whose planes belong to two images (different weights)
])
def test_long_line_kernel_plane_groups(shape, dtype):
    """Channel-shared weights over enough planes that the long-line kernel runs
    several planes per workgroup."""
    n, c, h, w = shape
    wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, shared=True, seed=71 + c)
    _say("long-line plane groups %s %s" % (shape, dtype))
    inp = make_inputs(wl, DEV)
    got, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"],
                                       workspace=G.forward4_workspace(inp["x"], wl.cw))
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "scan4lp_kernel", times["scan_kernel"]
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"])
    assert _err(got, ref) <= TOL[dtype]


@pytest.mark.parametrize("chunk", [0, 7])
@pytest.mark.parametrize("shared", [False, True])
@pytest.mark.parametrize("dtype,shape,bands", [
    ("f32", (1, 2, 520, 600), 10),    # segments of 128 positions, halos and bands of 64 steps; ragged last segments
    ("bf16", (1, 2, 520, 600), 5),    # segments of 256, halos and bands of 128
    ("bf16", (2, 3, 1024, 512), 8),   # 24 lines; the horizontal scans outlast the vertical ones
])
def test_banded_kernel(dtype, shape, bands, shared, chunk):
    """Very few long lines: each line split across workgroups, the scan run
    in bands of steps (one launch per band)."""
    n, c, h, w = shape
    wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, shared=shared, chunk=chunk, seed=81 + h + w)
    _say("banded %s %s shared=%s chunk=%d" % (shape, dtype, shared, chunk))
    inp = make_inputs(wl, DEV)
    m = torch.randn((4, c), device=DEV) if chunk else None
    got, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], chunk_len=chunk,
                                       workspace=G.forward4_workspace(inp["x"], wl.cw), merge=m)
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "scan4band_kernel", times["scan_kernel"]
    assert times["scan"]["launches"] == bands
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=chunk, merge=None if m is None else _np(m))
    assert _err(got, ref) <= TOL[dtype]


def test_forward4_closed_form_constant_input():
    # lambda = 1, x = c: every direction's h at scan step t is (t+1) c, so the
    # merged output is (H + W + 2) c everywhere, whatever the logits.
    wl = _wl(n=2, c=3, h=45, w=77, seed=3)
    inp = make_inputs(wl, DEV)
    x = torch.full_like(inp["x"], 0.25)
    lam = [torch.ones_like(l) for l in inp["lam"]]
    y = G.gspn_forward4(x, inp["logits"], lam)
    torch.cuda.synchronize()
    np.testing.assert_allclose(_np(y), (45 + 77 + 2) * 0.25, rtol=2e-6)


def test_empty_inputs_are_no_ops():
    x = torch.empty(0, 2, 8, 8, device=DEV)
    z = [torch.empty(0, 2, 3, 8, 8, device=DEV)] * 4
    l = [torch.empty(0, 2, 8, 8, device=DEV)] * 4
    y = G.gspn_forward4(x, z, l)
    torch.cuda.synchronize()
    assert y.shape == x.shape


def test_deterministic():
    wl = _wl(n=2, c=4, h=50, w=60, seed=21)
    inp = make_inputs(wl, DEV)
    a = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"])
    b = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape,shared,kernel,expect", [
    # planes of at most 64 x 64: one pass, nothing else
    ((2, 3, 40, 56), False, "plane4_kernel", {"transpose": 0, "scan": 1, "combine": 0, "normalize": 0}),
    ((2, 3, 64, 64), True, "plane4_kernel", {"transpose": 0, "scan": 1, "combine": 0, "normalize": 0}),
    # few planes, lines whose 16-byte vectors fit 256 lanes: long-line kernel
    ((1, 2, 40, 72), False, "scan4lp_kernel", {"transpose": 1, "scan": 1, "combine": 1, "normalize": 0}),
    # channel-shared weights over several channels: normalised once per direction
    ((1, 3, 40, 72), True, "scan4lp_kernel", {"transpose": 1, "scan": 1, "combine": 1, "normalize": 4}),
    # few planes, lines not a whole number of vectors: one workgroup per line
    ((1, 2, 40, 70), False, "scan4v_kernel", {"transpose": 1, "scan": 1, "combine": 1, "normalize": 0}),
    # many planes: still one fused launch
    ((8, 80, 8, 72), False, "scan4lp_kernel", {"transpose": 1, "scan": 1, "combine": 1, "normalize": 0}),
    # lines longer than the fused launch takes: one launch per direction
    ((1, 1, 40, 2100), False, "scan_kernel", {"transpose": 1, "scan": 4, "combine": 1, "normalize": 0}),
])
def test_forward4_timed_matches_untimed(shape, shared, kernel, expect):
    n, c, h, w = shape
    wl = _wl(n=n, c=c, h=h, w=w, shared=shared, seed=31)
    _say("forward4_timed %s shared=%s" % (shape, shared))
    inp = make_inputs(wl, DEV)
    ws = G.forward4_workspace(inp["x"], wl.cw)
    a = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], workspace=ws)
    b, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert times["scan_kernel"] == kernel, times
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"])
    assert _err(b, ref) <= TOL["f32"]
    for stage, count in expect.items():
        assert times[stage]["launches"] == count, (stage, times)
        assert (times[stage]["ms"] > 0) == (count > 0), (stage, times)
    assert times["project_down"]["launches"] == 0 and times["project_up"]["launches"] == 0
    # without a workspace: four scans and nothing else (one pass for small planes)
    _, t2 = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"])
    nscan = 1 if kernel == "plane4_kernel" else 4
    assert t2["scan"]["launches"] == nscan
    assert sum(v["launches"] for k, v in t2.items() if k not in ("scan_kernel", "adjoint_plan")) == nscan


def test_proxy_forward4_timed_matches_untimed():
    wl = _wl(n=1, c=40, h=40, w=72, dtype="bf16", shared=True, seed=32, cp=8)
    _say("proxy_forward4_timed")
    inp = make_inputs(wl, DEV)
    ws = G.proxy_forward4_workspace(inp["x"], 8, 1)
    a = G.gspn_proxy_forward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"], workspace=ws)
    b, times = G.gspn_proxy_forward4_timed(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"],
                                           workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert times["project_down"]["launches"] == 1 and times["project_up"]["launches"] == 1
    assert times["scan"]["launches"] == 1 and times["scan_kernel"] == "scan4lp_kernel"
    assert times["normalize"]["launches"] == 1  # bf16 half pairs: four directions in one launch


# ----------------------------------------------------------------------------
# Proxy pipeline, small
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(1, 40, 33, 47, 8), (2, 64, 32, 64, 8), (1, 24, 64, 48, 4)])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_proxy_forward4_small(shape, dtype):
    n, c, h, w, cp = shape
    for shared in (True, False):
        wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, shared=shared, seed=13 + h, cp=cp)
        _say("proxy %s %s shared=%s" % (shape, dtype, shared))
        inp = make_inputs(wl, DEV)
        got = G.gspn_proxy_forward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"])
        torch.cuda.synchronize()
        ref = oracle.proxy_forward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"])
        assert _err(got, ref) <= TOL[dtype]


# ----------------------------------------------------------------------------
# Full-size workloads, in the launch configuration the bench times
# ----------------------------------------------------------------------------

def _plane_inputs(inp, wl, n, c):
    """CPU fp64 copies of the inputs of one (n, c) plane."""
    x = _np(inp["x"][n:n + 1, c:c + 1])
    wc = 0 if wl.shared_w else c
    zs = [_np(z[n:n + 1, wc:wc + 1]) for z in inp["logits"]]
    ls = [_np(l[n:n + 1, c:c + 1]) for l in inp["lam"]]
    return x, zs, ls


@pytest.mark.parametrize("name", ["tstage", "tstage_chunk8"])
def test_full_tstage(name):
    wl = WORKLOADS[name]
    _say("full %s" % name)
    inp = make_inputs(wl, DEV)
    got = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=wl.chunk,
                          workspace=G.forward4_workspace(inp["x"], wl.cw))
    torch.cuda.synchronize()
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], chunk=wl.chunk)
    assert _err(got, ref) <= TOL[wl.dtype]


@pytest.mark.parametrize("name,planes", [
    ("profile", [(0, 0), (7, 3), (15, 7)]),
    ("wide", [(0, 0), (0, 577), (0, 1151)]),
])
def test_full_size_sampled_planes(name, planes):
    wl = WORKLOADS[name]
    _say("full %s" % name)
    inp = make_inputs(wl, DEV)
    got = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], chunk_len=wl.chunk,
                          workspace=G.forward4_workspace(inp["x"], wl.cw))
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    for n, c in planes:
        x, zs, ls = _plane_inputs(inp, wl, n, c)
        ref = oracle.forward4(x, zs, ls, chunk=wl.chunk)
        e = _err(got[n:n + 1, c:c + 1], ref)
        _say("  plane (%d, %d): normwise error %.3g" % (n, c, e))
        assert e <= TOL[wl.dtype]


def test_full_size_wide_merge_sampled_planes():
    """The 1152-channel workload with learnable merge weights: the first 1024
    planes on the plane-sequential kernel, the last 128 (the tail) on the
    concurrent path, whose transposing merge reads the tail channels' merge
    weights in place; sampled planes from both against the oracle."""
    wl = WORKLOADS["wide"]
    _say("full wide, learnable merge")
    inp = make_inputs(wl, DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(wl.seed + 2000)
    m = torch.randn((4, wl.c), generator=g, device=DEV, dtype=torch.float32)
    got, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], chunk_len=wl.chunk,
                                       workspace=G.forward4_workspace(inp["x"], wl.cw), merge=m)
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "seq4_kernel" and times["tail"]["launches"] == 1, times
    mm = m.double().cpu().numpy()
    for c in (0, 1023, 1024, 1100, 1151):
        x, zs, ls = _plane_inputs(inp, wl, 0, c)
        ref = oracle.forward4(x, zs, ls, chunk=wl.chunk, merge=mm[:, c:c + 1])
        e = _err(got[0:1, c:c + 1], ref)
        _say("  channel %d: normwise error %.3g" % (c, e))
        assert e <= TOL[wl.dtype]


def test_full_size_no_workspace_sampled_planes():
    """The 1024^2, B=16, C=8 workload without a workspace: one launch per
    direction, horizontal lines as per-lane row tiles."""
    wl = WORKLOADS["profile"]
    _say("full profile, no workspace")
    inp = make_inputs(wl, DEV)
    got, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"], chunk_len=wl.chunk)
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "scan_kernel" and times["scan"]["launches"] == 4
    for n, c in [(0, 0), (9, 5)]:
        x, zs, ls = _plane_inputs(inp, wl, n, c)
        ref = oracle.forward4(x, zs, ls, chunk=wl.chunk)
        e = _err(got[n:n + 1, c:c + 1], ref)
        _say("  plane (%d, %d): normwise error %.3g" % (n, c, e))
        assert e <= TOL[wl.dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shared", [False, True])
def test_forward4_unaligned_views(dtype, shared):
    """Tensors that are element-aligned but not 16-byte aligned (views one
    element into a larger buffer): the vector kernels must step aside."""
    n, c, h, w = 1, 3, 40, 72
    wl = _wl(n=n, c=c, h=h, w=w, dtype=dtype, shared=shared, seed=51)
    inp = make_inputs(wl, DEV)

    def shifted(t):
        buf = torch.empty(t.numel() + 1, dtype=t.dtype, device=DEV)
        v = buf[1:].view(t.shape)
        v.copy_(t)
        return v

    x = shifted(inp["x"])
    zs = [shifted(z) for z in inp["logits"]]
    ls = [shifted(l) for l in inp["lam"]]
    out = shifted(torch.zeros_like(inp["x"]))
    got, times = G.gspn_forward4_timed(x, zs, ls, out=out, workspace=G.forward4_workspace(x, wl.cw))
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "scan4v_kernel", times["scan_kernel"]
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"])
    assert _err(got, ref) <= TOL[dtype]


def test_full_size_proxy_sampled_channels():
    wl = WORKLOADS["proxy"]
    _say("full proxy")
    inp = make_inputs(wl, DEV)
    got = G.gspn_proxy_forward4(inp["x"], inp["w_down"], inp["w_up"], inp["logits"], inp["lam"])
    torch.cuda.synchronize()
    assert torch.isfinite(got).all()
    # the oracle needs the whole proxy-space state: all 320 input channels
    xp = oracle.project(inp["x"], inp["w_down"])
    yp = oracle.forward4(xp, inp["logits"], inp["lam"])
    del xp
    chans = [0, 161, 319]
    ref = oracle.project(yp, _np(inp["w_up"])[chans])
    for j, c in enumerate(chans):
        e = _err(got[:, c:c + 1], ref[:, j:j + 1])
        _say("  channel %d: normwise error %.3g" % (c, e))
        assert e <= 2e-2


@pytest.mark.parametrize("shape,shared,merge,keep", [
    ((1, 17, 1024, 64), False, False, False),   # 1024-row horizontal lines, two column tiles
    ((2, 9, 1024, 96), False, True, False),     # three tiles, learnable merge, two images
    ((1, 20, 1024, 128), True, False, False),   # channel-shared fp32 weight triples
    ((1, 17, 1024, 64), False, False, True),    # the forward keeping its fp32 states
    ((1, 17, 960, 64), False, False, False),    # lines of 960 rows: the tile's last rounds unused
])
def test_long_line_column_tiles(shape, shared, merge, keep):
    """fp32 planes whose lines take one 256-lane workgroup: the long-line
    scan's horizontal directions read x through LDS column tiles (no
    transposed copy, no transpose launch) and match the oracle."""
    n, c, h, w = shape
    wl = _wl(n=n, c=c, h=h, w=w, dtype="f32", shared=shared, seed=61 + w + c)
    _say("column tiles %s shared=%s merge=%s keep=%s" % (shape, shared, merge, keep))
    inp = make_inputs(wl, DEV)
    m = None
    if merge:
        g = torch.Generator(device=DEV)
        g.manual_seed(3)
        m = torch.randn((4, c), generator=g, device=DEV)
    st = G.states_buffer(inp["x"]) if keep else None
    got, times = G.gspn_forward4_timed(inp["x"], inp["logits"], inp["lam"],
                                       workspace=G.forward4_workspace(inp["x"], wl.cw), merge=m, states=st)
    torch.cuda.synchronize()
    assert times["scan_kernel"] == "scan4lp_kernel", times["scan_kernel"]
    assert times["transpose"]["launches"] == 0, times
    ref = oracle.forward4(inp["x"], inp["logits"], inp["lam"], merge=None if m is None else _np(m))
    assert _err(got, ref) <= TOL["f32"]
    if keep:
        # the kept states are the four unweighted scans in their scan frames
        for d in range(4):
            hd = G.state_map(st, d, tuple(inp["x"].shape))
            rd = oracle.scan(d, _np(inp["x"]), _np(inp["logits"][d]), _np(inp["lam"][d]), 0)
            rd = rd if d < 2 else rd.transpose(0, 1, 3, 2)   # the oracle's map is in the array frame
            assert oracle.normwise_error(_np(hd), rd) <= TOL["f32"], d
