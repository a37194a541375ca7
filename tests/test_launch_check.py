"""Host-side replay of the library's launches (no GPU): libgspn_check.so is
the library's host code built with GSPN_CHECK_LAUNCHES, in which each
launcher replays its kernel's accesses block by block and thread by thread,
with the index functions the kernel itself calls, and checks every access
against the buffer that holds the pointer it goes through; the launch itself
only records the kernel, grid, block and LDS size.

The buffers are address ranges registered with the checker (nothing is
allocated or touched), sized as the Python binding sizes them: its
forward4_workspace, states_buffer and backward4_workspace(with_states=True)
on meta tensors.

The central case is the training step on the 64 x 96 x 56 x 56 stage map that
keeps the forward's fp32 states for the backward, a configuration that once
ended in a GPU memory fault.  Its replay showed the cause: lanes past the end
of a line computed their left neighbour's state offset without clamping it
into the line, and on the last row of the last plane of the last direction's
map that read up to 7 floats past the states buffer (whose size there, 147 x
2 MiB, leaves the allocator no slack).  The clamp is now in adj_left."""
import ctypes
import os

import pytest
import torch

from linear_spatial_propagation_gspn_amd import build as hipbuild
from linear_spatial_propagation_gspn_amd import gspn as G


_vp4 = ctypes.c_void_p * 4
_i64 = ctypes.c_int64


@pytest.fixture(scope="module")
def chk():
    src = os.path.join(hipbuild.CSRC)
    newest = max(os.path.getmtime(os.path.join(src, f)) for f in os.listdir(src))
    if not os.path.exists(hipbuild.CHECK_LIB) or os.path.getmtime(hipbuild.CHECK_LIB) < newest:
        hipbuild.build_check()
    lib = ctypes.CDLL(hipbuild.CHECK_LIB)
    lib.gspn_check_add_buffer.argtypes = [ctypes.c_char_p, ctypes.c_uint64, ctypes.c_uint64]
    lib.gspn_check_violations.restype = _i64
    lib.gspn_check_accesses.restype = _i64
    lib.gspn_check_launches.restype = _i64
    lib.gspn_check_report.restype = _i64
    lib.gspn_check_report.argtypes = [ctypes.c_char_p, _i64]
    for f in ("gspn_forward4", "gspn_backward4", "gspn_forward4_noalloc", "gspn_proxy_forward4", "gspn_proxy_backward4"):
        getattr(lib, f).restype = ctypes.c_int
    return lib


def report(lib) -> str:
    n = lib.gspn_check_report(None, 0)
    buf = ctypes.create_string_buffer(int(n) + 1)
    lib.gspn_check_report(buf, n + 1)
    return buf.value.decode()


class Space:
    """Disjoint address ranges registered as buffers, 2^36 bytes apart (so an
    overrun lands in no buffer) and 256-byte aligned."""

    def __init__(self, lib):
        self.lib = lib
        self.next = 1 << 44
        lib.gspn_check_reset()

    def buf(self, name: str, nbytes: int) -> int:
        assert 0 < nbytes < (1 << 36)
        base = self.next
        self.next += 1 << 36
        assert self.lib.gspn_check_add_buffer(name.encode(), base, nbytes) == 0
        return base


def _meta(n, c, h, w, dtype):
    return torch.empty((n, c, h, w), dtype=dtype, device="meta")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def training_step(lib, n, c, h, w, dtype=torch.float32, shared=False, chunk=0, merge=False, layout="scan",
                  keep_states=True, short_states=0):
    """Forward keeping the states, then the backward from them, through the
    check library's C ABI; returns the two status codes."""
    sp = Space(lib)
    x = _meta(n, c, h, w, dtype)
    es = x.element_size()
    cw = 1 if shared else c
    dt = G._dtype_code(x)
    lc = G._layout_code(layout)
    xb = n * c * h * w * es
    zb = n * cw * 3 * h * w * es
    px = sp.buf("x", xb)
    pz = [sp.buf("logits%d" % d, zb) for d in range(4)]
    pl = [sp.buf("lambda%d" % d, xb) for d in range(4)]
    py = sp.buf("y", xb)
    pm = sp.buf("merge", 4 * c * 4) if merge else None
    ps = sp.buf("states", _nbytes(G.states_buffer(x)) - short_states) if keep_states else None
    fws = G.forward4_workspace(x, cw, layout=layout)
    pw = sp.buf("forward workspace", _nbytes(fws))
    rf = lib.gspn_forward4(_i64(n), _i64(c), _i64(h), _i64(w), _i64(cw), _i64(chunk), ctypes.c_void_p(px),
                           _vp4(*pz), _vp4(*pl), ctypes.c_void_p(pm), ctypes.c_void_p(py), ctypes.c_void_p(ps),
                           ctypes.c_void_p(pw), _i64(_nbytes(fws)), dt, lc, None)
    pg = sp.buf("dL/dy", xb)
    pdx = sp.buf("dx", xb)
    pdz = [sp.buf("dlogits%d" % d, zb) for d in range(4)]
    pdl = [sp.buf("dlambda%d" % d, xb) for d in range(4)]
    pdm = sp.buf("dmerge", 4 * c * 4) if merge else None
    bws = G.backward4_workspace(x, cw, with_states=keep_states, layout=layout)
    pb = sp.buf("backward workspace", _nbytes(bws))
    rb = lib.gspn_backward4(_i64(n), _i64(c), _i64(h), _i64(w), _i64(cw), _i64(chunk), ctypes.c_void_p(px),
                            _vp4(*pz), _vp4(*pl), ctypes.c_void_p(pm), ctypes.c_void_p(ps), ctypes.c_void_p(pg),
                            ctypes.c_void_p(pdx), _vp4(*pdz), _vp4(*pdl), ctypes.c_void_p(pdm), ctypes.c_void_p(pb),
                            _i64(_nbytes(bws)), dt, lc, None)
    return rf, rb


def _kernels(text: str) -> list:
    return [line.split()[1] for line in text.splitlines() if line.startswith("launch ")]


def test_tstage_training_step_with_kept_states(chk):
    """The step that faulted: 64 x 96 x 56 x 56, fp32, per-channel logits,
    forward keeping its states, backward from them with the binding's
    shrunken workspace.  Every access of every launch stays in its buffer."""
    rf, rb = training_step(chk, 64, 96, 56, 56)
    text = report(chk)
    print(text)
    assert (rf, rb) == (0, 0), text
    assert _kernels(text) == [
        "transpose_kernel<float>", "(scan4lp_kernel<T,", "(combine_kernel<float,",      # forward
        "transpose_kernel<float>", "transpose_kernel<float>", "(adj4_kernel<float,", "(combine_kernel<float,",
    ], text
    assert chk.gspn_check_violations() == 0, text
    # every position of the four directions, every step: far more than 10^9 accesses
    assert chk.gspn_check_accesses() > 10 ** 9


@pytest.mark.parametrize("case", [
    dict(n=2, c=3, h=23, w=41, chunk=5),                          # ragged lines, element tiles
    dict(n=1, c=5, h=40, w=72, dtype=torch.bfloat16, shared=True),  # channel groups of three, the last ragged
    dict(n=1, c=2, h=64, w=64, merge=True, chunk=7),
    dict(n=1, c=3, h=56, w=56, layout="array"),
])
def test_small_plane_steps_with_kept_states(chk, case):
    case = dict(case)
    rf, rb = training_step(chk, case.pop("n"), case.pop("c"), case.pop("h"), case.pop("w"), **case)
    text = report(chk)
    assert (rf, rb) == (0, 0), text
    assert chk.gspn_check_violations() == 0, text


@pytest.mark.parametrize("case", [
    dict(n=1, c=2, h=200, w=130, chunk=9),
    dict(n=1, c=9, h=64, w=128, dtype=torch.bfloat16, shared=True),
    dict(n=1, c=2, h=72, w=1500),                                 # two positions per lane in the adjoint
])
def test_long_line_steps(chk, case):
    """Steps of planes above 64 x 64 (kept states are supported there)."""
    case = dict(case)
    rf, rb = training_step(chk, case.pop("n"), case.pop("c"), case.pop("h"), case.pop("w"), **case)
    text = report(chk)
    assert (rf, rb) == (0, 0), text
    assert chk.gspn_check_violations() == 0, text


def test_checker_sees_an_overrun(chk):
    """A states buffer one float short: the replay of the forward's scan (its
    last plane's store) and of the backward's adjoint must report it."""
    rf, rb = training_step(chk, 2, 3, 40, 48, short_states=4)
    text = report(chk)
    assert (rf, rb) == (0, 0)
    assert chk.gspn_check_violations() > 0
    assert "scan4lp_kernel" in text and "adj4_kernel" in text


def test_unreplayed_launch_is_reported(chk):
    """The plane-resident forward has no host replay: its launch is reported
    rather than passed over."""
    sp = Space(chk)
    n, c, h, w = 1, 2, 16, 16
    xb = n * c * h * w * 4
    px = sp.buf("x", xb)
    pz = [sp.buf("logits%d" % d, 3 * xb) for d in range(4)]
    pl = [sp.buf("lambda%d" % d, xb) for d in range(4)]
    py = sp.buf("y", xb)
    r = chk.gspn_forward4(_i64(n), _i64(c), _i64(h), _i64(w), _i64(c), _i64(0), ctypes.c_void_p(px), _vp4(*pz),
                          _vp4(*pl), None, ctypes.c_void_p(py), None, None, _i64(0), 0, 0, None)
    assert r == 0
    assert chk.gspn_check_violations() == 1
    assert "plane4_kernel" in report(chk) and "without a host replay" in report(chk)


def test_allocation_free_forward_stays_in_its_scratch(chk):
    """gspn_forward4_noalloc works in the library's static scratch array; the
    checking build stands an address range in for it, registered here at the
    array's size: the transposes, scans and merge stay inside it."""
    sp = Space(chk)
    assert chk.gspn_check_add_buffer(b"scratch", 0x7E << 40, 64 << 20) == 0
    n, c, h, w = 1, 3, 200, 130
    xb = n * c * h * w * 4
    px = sp.buf("x", xb)
    pz = [sp.buf("logits%d" % d, 3 * xb) for d in range(4)]
    pl = [sp.buf("lambda%d" % d, xb) for d in range(4)]
    py = sp.buf("y", xb)
    for layout in (0, 1):
        r = chk.gspn_forward4_noalloc(_i64(n), _i64(c), _i64(h), _i64(w), _i64(c), _i64(9), ctypes.c_void_p(px),
                                      _vp4(*pz), _vp4(*pl), None, ctypes.c_void_p(py), None, 0, layout, None)
        assert r == 0
    text = report(chk)
    assert chk.gspn_check_violations() == 0, text
    assert "scan4v_kernel" in text and "combine_kernel" in text


def _random_cases(seed: int, count: int):
    """Random shapes for the replayed paths: planes above 64 x 64 in one
    dimension, lines up to 2048 (so the four-direction kernels run), mixed
    dtypes, chunk lengths, shared logits, merge weights and layouts."""
    import random
    rng = random.Random(seed)
    out = []
    while len(out) < count:
        h = rng.choice([1, 2, 3, 7, 17, 33, 64, 65, 96, 130, 257, 520, 1025, 2048])
        w = rng.choice([1, 5, 31, 63, 65, 100, 128, 333, 1000, 1023, 1536, 2048])
        if h <= 64 and w <= 64:
            continue
        n = rng.choice([1, 2])
        c = rng.choice([1, 2, 3, 5, 9])
        if n * c * h * w > 3_000_000:
            continue
        out.append(dict(n=n, c=c, h=h, w=w, dtype=rng.choice([torch.float32, torch.bfloat16]),
                        shared=rng.random() < 0.4, chunk=rng.choice([0, 0, 1, 3, 8, 100]),
                        merge=rng.random() < 0.3, layout=rng.choice(["scan", "scan", "array"]),
                        keep_states=rng.random() < 0.7))
    return out


@pytest.mark.parametrize("case", _random_cases(2026, 24), ids=lambda c: "%dx%dx%dx%d" % (c["n"], c["c"], c["h"], c["w"]))
def test_random_shapes_stay_in_bounds(chk, case):
    """Random shapes: forward (keeping the states or not) and backward,
    every replayed launch in bounds.  Launches without a replay (the banded
    scan of very few long lines) are allowed here and reported, not failed."""
    case = dict(case)
    rf, rb = training_step(chk, case.pop("n"), case.pop("c"), case.pop("h"), case.pop("w"), **case)
    text = report(chk)
    assert (rf, rb) == (0, 0), text
    bad = [l for l in text.splitlines() if l.startswith("violation") and "without a host replay" not in l]
    assert not bad, text


def proxy_training_step(lib, n, c, h, w, cp, dtype=torch.bfloat16, shared=True, chunk=0, merge=False, keep=False):
    """The compressive-proxy forward, then its backward, through the check
    library's C ABI (buffers sized as the binding sizes them); keep: the
    forward keeps the proxy-space state for the backward; returns the two
    status codes."""
    sp = Space(lib)
    x = _meta(n, c, h, w, dtype)
    es = x.element_size()
    cw = 1 if shared else cp
    dt = G._dtype_code(x)
    xb = n * c * h * w * es
    pb = n * cp * h * w * es
    zb = n * cw * 3 * h * w * es
    px = sp.buf("x", xb)
    pwd = sp.buf("w_down", cp * c * es)
    pwu = sp.buf("w_up", c * cp * es)
    pz = [sp.buf("logits%d" % d, zb) for d in range(4)]
    pl = [sp.buf("lambda%d" % d, pb) for d in range(4)]
    pm = sp.buf("merge", 4 * cp * 4) if merge else None
    py = sp.buf("y", xb)
    fws = G.proxy_forward4_workspace(x, cp, cw)
    pfw = sp.buf("forward workspace", _nbytes(fws))
    lib.gspn_proxy_states_bytes.restype = _i64
    pk = sp.buf("proxy states", lib.gspn_proxy_states_bytes(_i64(n), _i64(cp), _i64(h), _i64(w), dt)) if keep else None
    rf = lib.gspn_proxy_forward4(_i64(n), _i64(c), _i64(h), _i64(w), _i64(cp), _i64(cw), _i64(chunk),
                                 ctypes.c_void_p(px), ctypes.c_void_p(pwd), ctypes.c_void_p(pwu), _vp4(*pz), _vp4(*pl),
                                 ctypes.c_void_p(pm), ctypes.c_void_p(py), ctypes.c_void_p(pk), ctypes.c_void_p(pfw),
                                 _i64(_nbytes(fws)), dt, 0, None)
    pg = sp.buf("dL/dy", xb)
    pdx = sp.buf("dx", xb)
    pdwd = sp.buf("dw_down", cp * c * 4)
    pdwu = sp.buf("dw_up", c * cp * 4)
    pdz = [sp.buf("dlogits%d" % d, zb) for d in range(4)]
    pdl = [sp.buf("dlambda%d" % d, pb) for d in range(4)]
    pdm = sp.buf("dmerge", 4 * cp * 4) if merge else None
    bws = G.proxy_backward4_workspace(x, cp, cw)
    pbw = sp.buf("backward workspace", _nbytes(bws))
    rb = lib.gspn_proxy_backward4(_i64(n), _i64(c), _i64(h), _i64(w), _i64(cp), _i64(cw), _i64(chunk),
                                  ctypes.c_void_p(px), ctypes.c_void_p(pwd), ctypes.c_void_p(pwu), _vp4(*pz),
                                  _vp4(*pl), ctypes.c_void_p(pm), ctypes.c_void_p(pk), ctypes.c_void_p(pg),
                                  ctypes.c_void_p(pdx),
                                  ctypes.c_void_p(pdwd), ctypes.c_void_p(pdwu), _vp4(*pdz), _vp4(*pdl),
                                  ctypes.c_void_p(pdm), ctypes.c_void_p(pbw), _i64(_nbytes(bws)), dt, 0, None)
    return rf, rb


@pytest.mark.parametrize("case", [
    dict(n=1, c=320, h=64, w=256, cp=8),                                  # folded projection, ten channel blocks
    dict(n=2, c=328, h=32, w=128, cp=5, merge=True),                      # two channel groups, projection apart
    dict(n=1, c=24, h=70, w=100, cp=3, chunk=9),                          # bf16, ragged pixel count: VALU sums
    dict(n=2, c=7, h=65, w=66, cp=2, dtype=torch.float32, shared=False),  # fp32
], ids=["fold", "groups", "ragged", "f32"])
def test_proxy_backward_stays_in_bounds(chk, case):
    """The compressive-proxy backward: the weight transposes, the fused
    projection with the weight-gradient partial sums, the VALU partial sums
    and the fixed-order reduction stay inside their buffers.  The
    projections and the banded scan have no host replay; their launches are
    reported, not failed."""
    case = dict(case)
    rf, rb = proxy_training_step(chk, case.pop("n"), case.pop("c"), case.pop("h"), case.pop("w"), case.pop("cp"),
                                 **case)
    text = report(chk)
    assert (rf, rb) == (0, 0), text
    bad = [l for l in text.splitlines() if l.startswith("violation") and "without a host replay" not in l]
    assert not bad, text
    kernels = set(_kernels(text))
    assert "wgrad_reduce_kernel" in " ".join(kernels), text


@pytest.mark.parametrize("case", [
    dict(n=1, c=320, h=64, w=256, cp=8),                                  # planes > 64 x 64: the scans kept too
    dict(n=2, c=7, h=40, w=48, cp=2, dtype=torch.float32, shared=False),  # small planes: x_p and y_p only
], ids=["scans", "small"])
def test_proxy_training_step_with_kept_states_stays_in_bounds(chk, case):
    """The compressive-proxy forward keeping its proxy-space state in a
    buffer of gspn_proxy_states_bytes, the backward reading it instead of
    recomputing: every replayed launch stays inside its buffers, and the
    backward launches neither the down projection nor a forward scan."""
    base = dict(case)
    case = dict(case)
    rf, rb = proxy_training_step(chk, case.pop("n"), case.pop("c"), case.pop("h"), case.pop("w"), case.pop("cp"),
                                 keep=True, **case)
    text = report(chk)
    assert (rf, rb) == (0, 0), text
    bad = [l for l in text.splitlines() if l.startswith("violation") and "without a host replay" not in l]
    assert not bad, text
    kept = _kernels(text)
    rf, rb = proxy_training_step(chk, base.pop("n"), base.pop("c"), base.pop("h"), base.pop("w"), base.pop("cp"),
                                 **base)
    assert (rf, rb) == (0, 0)
    full = _kernels(report(chk))
    # the same launches but the backward's recompute: one projection (x down)
    # and the proxy-space forward fewer
    proj = lambda ks: sum(1 for k in ks if "project" in k and "wgrad" not in k)
    assert proj(kept) == proj(full) - 1, (kept, full)
    assert len(kept) < len(full) - 1, (kept, full)


@pytest.mark.parametrize("case", [
    dict(n=1, c=2, h=520, w=512, dtype=torch.bfloat16, shared=True, merge=True, keep_states=False),
    dict(n=2, c=1, h=512, w=600, dtype=torch.float32, keep_states=True),
    dict(n=1, c=3, h=700, w=530, dtype=torch.bfloat16, layout="array", keep_states=False),
], ids=["bf16-shared-merge", "f32-states", "bf16-array"])
def test_banded_adjoint_stays_in_bounds(chk, case):
    """Very few long lines: the backward runs the banded adjoint (segments
    with halos, one launch per band of steps); every band's loads, the
    products it reads from the band above and writes for the band below,
    and the segment's own stores stay inside their buffers."""
    case = dict(case)
    rf, rb = training_step(chk, case.pop("n"), case.pop("c"), case.pop("h"), case.pop("w"), **case)
    text = report(chk)
    assert (rf, rb) == (0, 0), text
    bad = [l for l in text.splitlines() if l.startswith("violation") and "without a host replay" not in l]
    assert not bad, text
    assert "adj4band_kernel" in text and "adj4_kernel<" not in text, text


def forward_only(lib, n, c, h, w, dtype=torch.float32):
    """The four-direction forward with the binding's workspace, no states."""
    sp = Space(lib)
    x = _meta(n, c, h, w, dtype)
    es = x.element_size()
    xb = n * c * h * w * es
    px = sp.buf("x", xb)
    pz = [sp.buf("logits%d" % d, 3 * xb) for d in range(4)]
    pl = [sp.buf("lambda%d" % d, xb) for d in range(4)]
    py = sp.buf("y", xb)
    fws = G.forward4_workspace(x, c)
    pw = sp.buf("forward workspace", _nbytes(fws))
    return lib.gspn_forward4(_i64(n), _i64(c), _i64(h), _i64(w), _i64(c), _i64(0), ctypes.c_void_p(px), _vp4(*pz),
                             _vp4(*pl), None, ctypes.c_void_p(py), None, ctypes.c_void_p(pw), _i64(_nbytes(fws)),
                             G._dtype_code(x), 0, None)


def _lp_dynamic_lds(text: str) -> int:
    lines = [l for l in text.splitlines() if l.startswith("launch ") and "scan4lp_kernel" in l]
    assert len(lines) == 1, text
    return int(lines[0].split("lds=")[1].split("+")[0])


@pytest.mark.parametrize("c, h, w, reserved", [
    (64, 8, 2048, True),    # four-wave workgroups, 256 of them: one whole round of one a CU
    (65, 8, 2048, False),   # 260: a second round nearly empty, so none reserved
    (64, 8, 512, False),    # one-wave workgroups (short lines): as many a CU as fit
])
def test_long_line_scan_lds_reservation(chk, c, h, w, reserved):
    """The long-line scan reserves LDS it does not use, so that one four-wave
    workgroup runs a CU (on the checking build's 256 CUs), only where the grid
    is whole rounds of them; the reservation leaves room for one workgroup,
    not two.  (bf16: fp32 planes of such lines read x through column tiles,
    whose static LDS leaves one workgroup a CU anyway.)"""
    assert forward_only(chk, 1, c, h, w, torch.bfloat16) == 0
    text = report(chk)
    assert chk.gspn_check_violations() == 0, text
    lds = _lp_dynamic_lds(text)
    if reserved:
        assert 80 * 1024 < lds <= 160 * 1024 - 1024, text
    else:
        assert lds == 0, text


@pytest.mark.parametrize("n, c, h, w, keep", [
    (1, 17, 1024, 64, False),    # 1024-row horizontal lines of 64 steps: two column tiles
    (1, 17, 1024, 96, True),     # three tiles, the states kept (fp32 maps written by the scan)
])
def test_long_line_scan_column_tiles(chk, n, c, h, w, keep):
    """fp32 planes whose lines take one 256-lane workgroup: the long-line
    scan's horizontal directions read x through LDS column tiles instead of a
    transposed copy (no transpose launch in the forward); every tile load
    and tile-row read stays in bounds, and the tile is the kernel's static
    LDS."""
    if keep:
        rf, rb = training_step(chk, n, c, h, w)
        assert (rf, rb) == (0, 0)
    else:
        assert forward_only(chk, n, c, h, w) == 0
    text = report(chk)
    assert chk.gspn_check_violations() == 0, text
    ks = _kernels(text)
    fwd = ks[:ks.index("(combine_kernel<float,") + 1]
    assert "transpose_kernel<float>" not in fwd, text
    lines = [l for l in text.splitlines() if l.startswith("launch ") and "scan4lp_kernel" in l]
    dyn, static = (int(v) for v in lines[0].split("lds=")[1].split("+"))
    assert dyn == 0 and static > 128 * 1024, text   # the column tile is static LDS; nothing reserved
