"""GPU parity of the backward pass: gspn_backward4 (through the C ABI) against
the fp64 oracle's gradient on the same seeded inputs and the same seeded
dL/dy.  Tolerances are the forward's, normwise per output tensor: 1e-5 for
fp32 storage, 2e-2 for bf16 storage."""
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
    t = torch.randn((wl.n, wl.c_scan, wl.h, wl.w), generator=g, device=DEV, dtype=torch.float32)
    return t.to(wl.torch_dtype)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    G.lib()
    yield
    torch.cuda.synchronize()


def _check_all(got, ref, tol, label):
    dx, dz, dl = got
    rdx, rdl, rdz = ref
    errs = {"dx": oracle.normwise_error(_np(dx), rdx)}
    for d in range(4):
        errs["dlam%d" % d] = oracle.normwise_error(_np(dl[d]), rdl[d])
        errs["dlogits%d" % d] = oracle.normwise_error(_np(dz[d]), rdz[d])
    worst = max(errs.values())
    _say("  %s: worst normwise error %.3g" % (label, worst))
    assert worst <= tol, errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunk", [0, 5])
@pytest.mark.parametrize("shape,shared", [
    ((1, 2, 16, 16), False),
    ((2, 3, 23, 41), False),
    ((1, 2, 40, 72), True),
    ((1, 1, 70, 37), False),
    ((1, 2, 5, 1000), False),     # one position per lane, 16 waves
    ((1, 1, 3, 1500), True),      # two positions per lane
    ((2, 3, 9, 1), False),        # lines of length 1 / single-step scans
    ((1, 3, 30, 50), True),       # plane-resident adjoint, shared-logit sums over channels
    ((1, 2, 64, 64), False),      # the largest plane-resident plane
    ((2, 2, 1, 7), False),        # a single line per plane
    ((1, 2, 17, 1), True),        # a single column per plane
    ((1, 3, 1, 1), True),         # one-position planes: no neighbours, centre weight 1
    ((2, 37, 24, 72), True),      # shared logits summed over ten channel groups, the last one ragged
    ((1, 37, 20, 30), True),      # the same over 37 plane-resident workgroups
])
def test_backward_small(shape, shared, chunk, dtype):
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, chunk, 300 + h + w)
    _say("backward %s shared=%s chunk=%d %s" % (shape, shared, chunk, dtype))
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 17)
    got = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk)
    torch.cuda.synchronize()
    ref = oracle.backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk=chunk)
    _check_all(got, ref, TOL[dtype], "all outputs")


def test_backward_timed_matches_untimed():
    wl = Workload("case", 1, 3, 40, 72, "bf16", True, 0, 12)
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 4)
    a = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy)
    t = G.StageTimes()
    b = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, times=t)
    torch.cuda.synchronize()
    st = t.as_dict()
    assert st["transpose"]["launches"] == 2 and st["scan"]["launches"] == 1
    assert st["normalize"]["launches"] == 1       # shared logits normalised once, four directions in one launch
    assert st["adjoint"]["launches"] == 1 and st["combine"]["launches"] == 1
    assert st["reduce"]["launches"] == 5          # clear the sums, store four directions
    assert st["adjoint"]["ms"] > 0
    assert torch.equal(a[0], b[0])
    for d in range(4):
        assert torch.equal(a[2][d], b[2][d])
        # shared-logit sums are fp32 atomics: equal up to their summation order
        assert torch.allclose(a[1][d].float(), b[1][d].float(), rtol=2e-2, atol=1e-2)


def test_backward_deterministic_per_channel():
    wl = Workload("case", 2, 3, 30, 50, "f32", False, 0, 9)
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 3)
    a = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy)
    b = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0])
    for d in range(4):
        assert torch.equal(a[1][d], b[1][d]) and torch.equal(a[2][d], b[2][d])


def test_backward_full_profile_sampled_planes():
    """The 1024^2, B=16, C=8 workload: the call on the whole batch, checked on
    sampled planes that the oracle computes on their own (per-channel logits,
    so every plane's gradient is independent)."""
    wl = WORKLOADS["profile"]
    _say("backward full profile")
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 23)
    dx, dz, dl = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy)
    torch.cuda.synchronize()
    assert torch.isfinite(dx).all()
    for n, c in [(0, 0), (15, 7)]:
        sl = (slice(n, n + 1), slice(c, c + 1))
        ref = oracle.backward4(inp["x"][sl], [z[sl] for z in inp["logits"]], [l[sl] for l in inp["lam"]],
                               gy[sl])
        got = (dx[sl], [z[sl] for z in dz], [l[sl] for l in dl])
        _check_all(got, ref, TOL["f32"], "plane (%d, %d)" % (n, c))


def test_backward_full_tstage_sampled_planes():
    """The 64 x 96 x 56 x 56 stage map (plane-resident backward): the call
    on the whole batch, checked on sampled planes that the oracle computes on
    their own."""
    wl = WORKLOADS["tstage"]
    _say("backward full tstage")
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 29)
    t = G.StageTimes()
    dx, dz, dl = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, times=t)
    torch.cuda.synchronize()
    st = t.as_dict()
    assert st["scan_kernel"] == "plane4_kernel"
    # one launch: the adjoint recomputes the forward states itself
    assert st["scan"]["launches"] == 0 and st["adjoint"]["launches"] == 1
    assert st["transpose"]["launches"] == 0 and st["combine"]["launches"] == 0
    assert torch.isfinite(dx).all()
    for n, c in [(0, 0), (63, 95), (17, 40)]:
        sl = (slice(n, n + 1), slice(c, c + 1))
        ref = oracle.backward4(inp["x"][sl], [z[sl] for z in inp["logits"]], [l[sl] for l in inp["lam"]],
                               gy[sl])
        got = (dx[sl], [z[sl] for z in dz], [l[sl] for l in dl])
        _check_all(got, ref, TOL["f32"], "plane (%d, %d)" % (n, c))


WIDE_PLAN = {"kernel": "adj4_kernel", "positions_per_lane": 1, "channel_group": 3, "nontemporal": True}


@pytest.mark.parametrize("chunk", [0, 5])
@pytest.mark.parametrize("shape", [(1, 10, 64, 128), (1, 10, 64, 1024), (1, 10, 128, 1024)])
def test_backward_shared_groups_of_three_nontemporal(shape, chunk):
    """The wide workload's adjoint instance: bf16 storage, channel-shared
    logits summed over groups of three channels (10 = 3 + 3 + 3 + 1: the last
    group ragged), one position per lane on lines of up to 1024 positions, and the
    non-temporal streams that every line being a whole number of 128-byte
    cache lines selects (H and W multiples of 64)."""
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, "bf16", True, chunk, 700 + h + w)
    _say("backward groups of three %s chunk=%d" % (shape, chunk))
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 31)
    t = G.StageTimes()
    got = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk, times=t)
    torch.cuda.synchronize()
    assert t.as_dict()["adjoint_plan"] == WIDE_PLAN
    ref = oracle.backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk=chunk)
    _check_all(got, ref, TOL["bf16"], "all outputs")


def test_backward_full_wide_sampled_channels():
    """The 1024^2, B=1, C=1152 workload (bf16, channel-shared logits): the
    call on the whole tensor, in the configuration the bench times.  dx and
    every dlambda are checked on sampled channels, which the oracle computes
    on their own (with the shared logits).  The shared dlogits sum over all
    1152 channels; the gradient is linear in dL/dy, so a second call with
    dL/dy zero outside the sampled channels must give the oracle's dlogits of
    those channels alone, summed."""
    wl = WORKLOADS["wide"]
    _say("backward full wide")
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 37)
    t = G.StageTimes()
    dx, dz, dl = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, times=t)
    torch.cuda.synchronize()
    assert t.as_dict()["adjoint_plan"] == WIDE_PLAN
    assert torch.isfinite(dx).all()
    chans = [0, 577, 1151]
    zs = [_np(z) for z in inp["logits"]]
    for c in chans:
        sl = (slice(0, 1), slice(c, c + 1))
        rdx, rdl, _ = oracle.backward4(_np(inp["x"][sl]), zs, [_np(l[sl]) for l in inp["lam"]], _np(gy[sl]))
        errs = {"dx": oracle.normwise_error(_np(dx[sl]), rdx)}
        for d in range(4):
            errs["dlam%d" % d] = oracle.normwise_error(_np(dl[d][sl]), rdl[d])
        _say("  channel %d: worst normwise error %.3g" % (c, max(errs.values())))
        assert max(errs.values()) <= TOL["bf16"], errs
    gz = torch.zeros_like(gy)
    gz[:, chans] = gy[:, chans]
    _, dz2, _ = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gz, out=(dx, dz, dl))
    torch.cuda.synchronize()
    _, _, rdz = oracle.backward4(_np(inp["x"][:, chans]), zs, [_np(l[:, chans]) for l in inp["lam"]],
                                 _np(gz[:, chans]))
    for d in range(4):
        e = oracle.normwise_error(_np(dz2[d]), rdz[d])
        _say("  dlogits %d of channels %s: normwise error %.3g" % (d, chans, e))
        assert e <= TOL["bf16"]


@pytest.mark.parametrize("shape,shared,dtype,merge,keep", [
    ((1, 2, 512, 640), False, "f32", False, False),
    ((1, 3, 600, 520), True, "bf16", True, False),
    ((2, 2, 1030, 513), True, "f32", False, True),     # states kept by the forward
    ((1, 1, 2048, 512), False, "bf16", False, False),  # sixteen bands of the vertical scans, four of the horizontal
])
def test_backward_banded(shape, shared, dtype, merge, keep):
    """Very few long unchunked lines: the adjoint runs in bands of 128 steps
    over segments of 256 positions with 128-position halos (adj4band_kernel),
    one launch per band, and matches the oracle's gradient."""
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, dtype, shared, 0, 700 + h + w)
    _say("banded backward %s shared=%s %s merge=%s states=%s" % (shape, shared, dtype, merge, keep))
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 23)
    m = None
    if merge:
        g = torch.Generator(device=DEV)
        g.manual_seed(5)
        m = torch.randn((4, c), generator=g, device=DEV, dtype=torch.float32)
    st = None
    if keep:
        _, st = G.gspn_forward4(inp["x"], inp["logits"], inp["lam"], workspace=G.forward4_workspace(inp["x"], wl.cw),
                                merge=m, states=True)
    t = G.StageTimes()
    got = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, merge=m, states=st, times=t)
    torch.cuda.synchronize()
    td = t.as_dict()
    assert td["adjoint_plan"]["kernel"] == "adj4band_kernel", td["adjoint_plan"]
    assert td["adjoint"]["launches"] == (max(h, w) + 127) // 128
    ref = oracle.backward4(inp["x"], inp["logits"], inp["lam"], gy, merge=None if m is None else _np(m))
    _check_all(got[:3], ref[:3], TOL[dtype], "all outputs")
    if merge:
        e = oracle.normwise_error(_np(got[3]), ref[3])
        _say("  dmerge normwise error %.3g" % e)
        assert e <= TOL[dtype]


WIDE_MERGE_PLAN = dict(WIDE_PLAN, channel_group=2)


@pytest.mark.parametrize("chunk", [0, 5])
@pytest.mark.parametrize("shape", [(1, 9, 64, 128), (1, 9, 128, 1024)])
def test_backward_shared_merge_groups_of_two(shape, chunk):
    """The wide workload's adjoint with learnable merge weights: the same
    instance but for channel groups of two (9 = 2 + 2 + 2 + 2 + 1), which
    keep the merge's extra state in registers.  dx, every dlambda, every
    dlogits and dmerge against the oracle."""
    n, c, h, w = shape
    wl = Workload("case", n, c, h, w, "bf16", True, chunk, 750 + h + w)
    _say("backward merge groups of two %s chunk=%d" % (shape, chunk))
    inp = make_inputs(wl, DEV)
    gy = _gy(wl, 33)
    g = torch.Generator(device=DEV)
    g.manual_seed(wl.seed + 3)
    m = torch.randn((4, c), generator=g, device=DEV)
    t = G.StageTimes()
    got = G.gspn_backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk_len=chunk, merge=m, dmerge=True, times=t)
    torch.cuda.synchronize()
    assert t.as_dict()["adjoint_plan"] == WIDE_MERGE_PLAN
    ref = oracle.backward4(inp["x"], inp["logits"], inp["lam"], gy, chunk=chunk, merge=_np(m))
    _check_all(got[:3], ref[:3], TOL["bf16"], "all outputs")
    assert oracle.normwise_error(_np(got[3]), ref[3]) <= TOL["bf16"]
