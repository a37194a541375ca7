"""CPU tests of the C ABI: the library loads, exports every declared symbol,
and host-side validation rejects bad arguments before anything reaches a
device.  No call here passes validation with a non-empty tensor, so nothing
is ever launched (there is no GPU in this suite)."""
import ctypes
import os
import re

import pytest

from linear_spatial_propagation_gspn_amd import gspn as G

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gspn.h")

OK, NULLP, SHAPE, DIR, DTYPE, CHUNK, WCH, MISAL, ALIAS, UNSUP, HIP, WSPACE, LAYOUT = range(13)

# Fake, never-dereferenced device addresses (validation only compares them).
A = 0x10000000
B = 0x20000000
C_ = 0x30000000
D_ = 0x40000000
E_ = 0x50000000


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gspn_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return G.lib()


def test_library_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(G.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_abi_version_and_status_strings(lib):
    assert lib.gspn_abi_version() == 11
    for code in range(13):
        s = lib.gspn_status_string(code).decode()
        assert s.startswith(G.STATUS[code])
    assert lib.gspn_status_string(99).decode() == "unknown gspn_status"


def scan(lib, dir=0, chunk=0, n=1, c=2, h=8, w=8, cw=2, x=A, wts=B, logits=1, lam=C_, out=D_,
         acc=0, dt=0):
    return lib.gspn_scan_fwd(dir, chunk, n, c, h, w, cw, x, wts, logits, lam, out, acc, dt, None)


def test_scan_validation(lib):
    assert scan(lib, dt=2) == DTYPE
    assert scan(lib, dir=4) == DIR
    assert scan(lib, dir=-1) == DIR
    assert scan(lib, n=-1) == SHAPE
    assert scan(lib, h=1 << 31) == SHAPE
    assert scan(lib, n=1 << 20, c=1 << 20, h=1 << 20, w=1 << 10) == SHAPE  # > 2^58 elements
    assert scan(lib, chunk=-1) == CHUNK
    assert scan(lib, cw=3) == WCH
    assert scan(lib, c=1, cw=2) == WCH
    assert scan(lib, w=4097) == UNSUP                    # vertical line longer than the limit
    assert scan(lib, dir=2, h=4097, w=4) == UNSUP        # horizontal lines run along H
    assert scan(lib, x=0) == NULLP
    assert scan(lib, wts=0) == NULLP
    assert scan(lib, lam=0) == NULLP
    assert scan(lib, out=0) == NULLP
    assert scan(lib, x=A + 2) == MISAL
    assert scan(lib, dt=1, x=A + 1) == MISAL
    assert scan(lib, out=A) == ALIAS                     # out == x
    assert scan(lib, out=B + 64) == ALIAS                # inside the weights
    assert scan(lib, out=C_ + 4) == ALIAS                # inside lambda


def test_scan_empty_is_a_no_op(lib):
    # An empty tensor returns OK without looking at pointers (all NULL here).
    assert scan(lib, n=0, x=0, wts=0, lam=0, out=0) == OK
    assert scan(lib, h=0, x=0, wts=0, lam=0, out=0) == OK
    # ...but enum and chunk checks still run first.
    assert scan(lib, n=0, dir=7) == DIR


def test_forward4_validation(lib):
    vp4 = ctypes.c_void_p * 4
    zs = vp4(B, B + 0x1000000, B + 0x2000000, B + 0x3000000)
    ls = vp4(C_, C_, C_, C_)
    W = 0x60000000
    def states(planes, lmax):  # fp32 scan states at band boundaries, two buffers of four directions
        return 2 * 4 * planes * lmax * 4

    wsb = lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 2, 0, 0)
    assert wsb == 4 * 2 * 64 * 4 + states(2, 8)
    assert lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 2, 1, 0) == 4 * 2 * 64 * 2 + states(2, 8)
    # channel-shared weights add the four directions' fp32 weights
    assert lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 1, 0, 0) == (4 * 2 * 64 * 4 + 4 * 3 * 64 * 4  # fp32 triples
                                                                  + states(2, 8))
    assert lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 1, 1, 0) == (4 * 2 * 64 * 2 + 4 * 64 * 4      # half pairs
                                                                  + states(2, 8))
    assert lib.gspn_forward4_workspace_bytes(1, 1, 8, 8, 1, 0, 0) == 4 * 64 * 4 + states(1, 8)
    assert lib.gspn_forward4_workspace_bytes(1, 1, 3, 5, 1, 1, 0) == 4 * 15 * 2 + states(1, 5)
    assert lib.gspn_forward4_workspace_bytes(2, 3, 6, 40, 3, 1, 0) == 4 * 2 * 3 * 240 * 2 + states(6, 40)
    assert lib.gspn_forward4_workspace_bytes(1, -2, 8, 8, 2, 0, 0) == -1
    assert lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 3, 0, 0) == -1
    assert lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 2, 5, 0) == -1

    def f(n=1, c=2, h=8, w=8, cw=2, chunk=0, x=A, z=zs, l=ls, m=None, y=D_, s=None, ws=None, wsb=0, dt=0, lay=0):
        return lib.gspn_forward4(n, c, h, w, cw, chunk, x, z, l, m, y, s, ws, wsb, dt, lay, None)

    assert f(dt=3) == DTYPE
    assert f(cw=3) == WCH
    assert f(chunk=-2) == CHUNK
    assert f(x=0) == NULLP
    assert f(z=vp4(B, 0, B, B)) == NULLP
    assert f(y=A) == ALIAS
    assert f(y=C_) == ALIAS
    assert f(l=vp4(C_, C_, C_, C_ + 1)) == MISAL
    assert f(ws=W, wsb=wsb - 1) == WSPACE
    assert f(ws=W + 2, wsb=wsb) == MISAL
    assert f(dt=1, ws=W + 2, wsb=wsb) == MISAL         # the workspace holds fp32 weights
    assert f(ws=D_ - 100, wsb=wsb) == ALIAS          # workspace overlaps y
    assert f(ws=A + 4, wsb=wsb) == ALIAS             # workspace overlaps x
    M = 0x68000000                                   # merge weights, fp32 [4][c]
    assert f(m=M + 2) == MISAL
    assert f(m=D_ + 8) == ALIAS                      # y overlaps the merge weights
    assert f(m=W + 16, ws=W, wsb=wsb) == ALIAS       # the workspace overlaps them
    S = 0x6a000000                                   # fp32 forward states, 4 maps of n*c*h*w
    assert f(s=S + 2, ws=W, wsb=wsb) == MISAL        # planes of at most 64 x 64 keep states too
    wsb = lib.gspn_forward4_workspace_bytes(1, 2, 8, 80, 2, 0, 0)
    f0 = f

    def f(**kw):
        kw.setdefault("w", 80)
        return f0(**kw)

    assert f(s=S) == WSPACE                          # states need the workspace
    assert f(s=S, ws=W, wsb=wsb, h=3000) == UNSUP    # and lines the four-direction launch takes
    assert f(s=S + 2, ws=W, wsb=wsb) == MISAL
    assert f(s=D_ - 16, ws=W, wsb=wsb) == ALIAS      # states overlap y
    assert f(s=C_ + 8, ws=W, wsb=wsb) == ALIAS       # states overlap lam
    assert f(s=W + 64, ws=W, wsb=wsb) == ALIAS       # states in the workspace
    assert f(s=M, m=M + 64, ws=W, wsb=wsb) == ALIAS  # states overlap the merge weights
    assert f(n=0, x=0, z=None, l=None, y=0) == OK


def test_scan4_validation(lib):
    vp4 = ctypes.c_void_p * 4
    zs = vp4(B, B + 0x1000000, B + 0x2000000, B + 0x3000000)
    ls = vp4(C_, C_, C_, C_)
    outs = vp4(D_, D_ + 0x1000000, D_ + 0x2000000, D_ + 0x3000000)

    def f(n=1, c=2, h=8, w=8, cw=2, chunk=0, x=A, z=zs, l=ls, o=outs, dt=0):
        return lib.gspn_scan4_fwd(n, c, h, w, cw, chunk, x, z, l, o, dt, None)

    assert f(dt=2) == DTYPE
    assert f(chunk=-1) == CHUNK
    assert f(cw=5) == WCH
    assert f(h=2049) == UNSUP                        # longer than the fused kernel's lines
    # each direction's (plane, chunk) count fits a grid, the four together do not
    assert f(n=700000, c=1, cw=1, h=2048, w=2048, chunk=1) == UNSUP
    assert f(o=vp4(D_, 0, D_, D_)) == NULLP
    assert f(o=vp4(D_, D_ + 0x1000000, D_ + 0x2000000, D_ + 2)) == MISAL
    assert f(o=vp4(D_, D_ + 16, D_ + 0x2000000, D_ + 0x3000000)) == ALIAS   # outputs overlap
    assert f(o=vp4(D_, A, D_ + 0x2000000, D_ + 0x3000000)) == ALIAS         # output on x
    assert f(n=0, x=0, z=None, l=None, o=None) == OK


def test_proxy_forward4_validation(lib):
    vp4 = ctypes.c_void_p * 4
    zs = vp4(B, B + 0x1000000, B + 0x2000000, B + 0x3000000)
    ls = vp4(C_, C_ + 0x1000000, C_ + 0x2000000, C_ + 0x3000000)
    WD, WU, WS = 0x70000000, 0x71000000, 0x72000000
    need = lib.gspn_proxy_forward4_workspace_bytes(1, 6, 8, 8, 2, 1, 1, 0)
    assert need == 2 * 2 * 64 * 2 + lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 1, 1, 0)
    assert lib.gspn_proxy_forward4_workspace_bytes(1, 6, 8, 8, 0, 1, 1, 0) == -1
    assert lib.gspn_proxy_forward4_workspace_bytes(1, 6, 8, 8, 2, 3, 1, 0) == -1

    def f(n=1, c=6, h=8, w=8, cp=2, cw=1, chunk=0, x=A, wd=WD, wu=WU, z=zs, l=ls, m=None, y=D_, ws=WS, wsb=need,
          dt=1, lay=0, st=None):
        return lib.gspn_proxy_forward4(n, c, h, w, cp, cw, chunk, x, wd, wu, z, l, m, y, st, ws, wsb, dt, lay, None)

    assert f(dt=2) == DTYPE
    assert f(cp=-1) == SHAPE
    assert f(chunk=-1) == CHUNK
    assert f(cw=3) == WCH
    assert f(h=5000) == UNSUP
    assert f(ws=0) == NULLP
    assert f(wd=0) == NULLP
    assert f(wsb=need - 1) == WSPACE
    assert f(ws=WS + 2) == MISAL
    assert f(y=A + 64) == ALIAS
    assert f(ws=A - 16) == ALIAS
    assert f(m=0x73000001) == MISAL
    assert f(m=WS + 64) == ALIAS                     # merge weights inside the workspace
    assert f(st=0x7E000010) == MISAL                 # kept state: 256-byte alignment
    assert f(st=WS + 256) == ALIAS                   # kept state inside the workspace
    assert f(st=A - 256) == ALIAS                    # kept state over x
    assert f(n=0, x=0, wd=0, wu=0, z=None, l=None, y=0, ws=0) == OK


def test_normalize_merge_project_validation(lib):
    nw = lib.gspn_normalize_weights
    assert nw(0, 1, 1, 4, 4, A, B, 5, None) == DTYPE
    assert nw(9, 1, 1, 4, 4, A, B, 0, None) == DIR
    assert nw(0, -1, 1, 4, 4, A, B, 0, None) == SHAPE
    assert nw(0, 1, 1, 4, 4, 0, B, 0, None) == NULLP
    assert nw(0, 1, 1, 4, 4, A, A + 8, 0, None) == ALIAS
    assert nw(0, 1, 1, 4, 4, A, B + 2, 0, None) == MISAL
    assert nw(0, 0, 1, 4, 4, 0, 0, 0, None) == OK

    m4 = lib.gspn_merge4
    assert m4(A, B, C_, D_, E_, 10, 7, None) == DTYPE
    assert m4(A, B, C_, D_, E_, -1, 0, None) == SHAPE
    assert m4(A, 0, C_, D_, E_, 10, 0, None) == NULLP
    assert m4(A, B, C_, D_, D_ + 4, 10, 0, None) == ALIAS
    assert m4(A, B, C_, D_, E_ + 1, 10, 1, None) == MISAL
    assert m4(0, 0, 0, 0, 0, 0, 0, None) == OK

    pp = lib.gspn_proxy_project
    assert pp(1, 8, 4, 4, 2, A, B, C_, 9, None) == DTYPE
    assert pp(1, -8, 4, 4, 2, A, B, C_, 0, None) == SHAPE
    assert pp(1, 0, 4, 4, 2, A, B, C_, 0, None) == SHAPE
    assert pp(1, 8, 4, 4, 2, A, 0, C_, 0, None) == NULLP
    assert pp(1, 8, 4, 4, 2, A, B, A + 16, 0, None) == ALIAS
    assert pp(1, 8, 4, 4, 2, A, B, B, 0, None) == ALIAS
    assert pp(1, 8, 4, 4, 2, A + 2, B, C_, 0, None) == MISAL
    assert pp(1, 8, 4, 4, 0, 0, 0, 0, 0, None) == OK


def test_binding_rejects_mismatched_tensors():
    import torch
    x = torch.zeros(1, 2, 4, 4)
    with pytest.raises(ValueError):
        # CPU tensors never reach the library
        G.gspn_scan_fwd(0, x, torch.zeros(1, 2, 3, 4, 4), torch.zeros(1, 2, 4, 4))
    with pytest.raises(TypeError):
        G.gspn_merge4([x.double()] * 4)


def test_timed_variants_validate_like_untimed(lib):
    vp4 = ctypes.c_void_p * 4
    zs = vp4(B, B + 0x1000000, B + 0x2000000, B + 0x3000000)
    ls = vp4(C_, C_, C_, C_)
    t = G.StageTimes()
    for i in range(len(G.STAGES)):
        t.ms[i], t.launches[i] = 7.0, 7

    def f(n=1, c=2, h=8, w=8, cw=2, chunk=0, x=A, y=D_, dt=0, times=ctypes.byref(t)):
        return lib.gspn_forward4_timed(n, c, h, w, cw, chunk, x, zs, ls, None, y, None, None, 0, dt, 0, None, times)

    assert f(times=None) == NULLP
    assert f(dt=3) == DTYPE
    assert f(cw=3) == WCH
    assert f(y=A) == ALIAS
    t.scan_kernel = 7
    assert f(n=0, x=0, y=0) == OK
    assert list(t.ms) == [0.0] * len(G.STAGES) and list(t.launches) == [0] * len(G.STAGES)
    assert t.scan_kernel == 0

    WD, WU, WS = 0x70000000, 0x71000000, 0x72000000
    need = lib.gspn_proxy_forward4_workspace_bytes(1, 6, 8, 8, 2, 1, 1, 0)

    def g(n=1, cp=2, ws=WS, wsb=need, dt=1, times=ctypes.byref(t)):
        return lib.gspn_proxy_forward4_timed(n, 6, 8, 8, cp, 1, 0, A, WD, WU, zs, ls, None, D_, None, ws, wsb, dt, 0,
                                             None, times)

    assert g(times=None) == NULLP
    assert g(dt=2) == DTYPE
    assert g(wsb=need - 1) == WSPACE
    assert g(ws=0) == NULLP
    assert g(n=0) == OK


def test_backward4_validation(lib):
    vp4 = ctypes.c_void_p * 4
    zs = vp4(B, B + 0x1000000, B + 0x2000000, B + 0x3000000)
    ls = vp4(C_, C_ + 0x1000000, C_ + 0x2000000, C_ + 0x3000000)
    dzs = vp4(0x60000000, 0x61000000, 0x62000000, 0x63000000)
    dls = vp4(0x64000000, 0x65000000, 0x66000000, 0x67000000)
    GY, DX, WS = 0x70000000, 0x71000000, 0x72000000
    need = lib.gspn_backward4_workspace_bytes(1, 2, 8, 8, 2, 0, 0)
    assert need == 9 * 2 * 64 * 4
    assert lib.gspn_backward4_workspace_bytes(1, 3, 8, 8, 1, 1, 0) == (4 * 3 * 64 * 4 + 4 * 64 * 4 + 4 * 3 * 64 * 4 +
                                                                   5 * 3 * 64 * 2)
    assert lib.gspn_backward4_workspace_bytes(1, 2, 8, 8, 3, 0, 0) == -1

    def f(n=1, c=2, h=8, w=8, cw=2, chunk=0, x=A, m=None, s=None, gy=GY, dx=DX, dz=dzs, dl=dls, dm=None, ws=WS,
          wsb=need, dt=0, lay=0):
        return lib.gspn_backward4(n, c, h, w, cw, chunk, x, zs, ls, m, s, gy, dx, dz, dl, dm, ws, wsb, dt, lay, None)

    assert f(dt=2) == DTYPE
    assert f(chunk=-1) == CHUNK
    assert f(cw=3) == WCH
    assert f(h=3000) == UNSUP                      # longer lines than the recomputed forward takes
    assert f(n=700000, c=1, cw=1, h=2048, w=2048, chunk=1) == UNSUP   # four directions' workgroups overflow a grid
    assert f(ws=0) == NULLP
    assert f(gy=0) == NULLP
    assert f(dz=vp4(0x60000000, 0, 0x62000000, 0x63000000)) == NULLP
    assert f(wsb=need - 1) == WSPACE
    assert f(ws=WS + 2) == MISAL
    assert f(dx=A + 8) == ALIAS                     # dx on x
    assert f(dx=dls[1]) == ALIAS                    # dx on dlam[1]
    assert f(dx=WS + 64) == ALIAS                   # dx in the workspace
    M, DM = 0x68000000, 0x69000000                  # merge weights and their gradient, fp32 [4][c]
    assert f(m=M + 1) == MISAL
    assert f(dm=DM + 2) == MISAL
    assert f(m=M, dm=M + 4) == ALIAS                # dmerge on the merge weights
    assert f(dm=DX + 8) == ALIAS                    # dmerge on dx
    assert f(dm=WS + 8) == ALIAS                    # dmerge in the workspace
    assert f(m=dls[2] + 4) == ALIAS                 # an output on the merge weights
    S = 0x6a000000                                  # fp32 forward states, 4 maps of n*c*h*w
    assert f(s=S + 2) == MISAL                      # planes of at most 64 x 64 take states too
    need80 = lib.gspn_backward4_workspace_bytes(1, 2, 8, 80, 2, 0, 0)
    smaller = need80 - 16 * 2 * 8 * 80              # the states' room in the workspace is not needed
    assert f(w=80, wsb=smaller) == WSPACE           # without states it is
    assert f(w=80, s=S, wsb=smaller - 1) == WSPACE
    assert f(w=80, s=S + 2, wsb=smaller) == MISAL
    assert f(w=80, s=WS + smaller - 4, wsb=smaller) == ALIAS   # states in the workspace
    assert f(w=80, s=DX - 16, wsb=smaller) == ALIAS       # dx on the states
    assert f(w=80, s=dzs[3] + 4, wsb=smaller) == ALIAS    # dlogits on the states
    assert f(w=80, s=0x6b000000, dm=0x6b000000 + 8, wsb=smaller) == ALIAS   # dmerge on the states
    assert f(n=0, x=0, gy=0, dx=0, dz=None, dl=None, ws=0) == OK
    t = G.StageTimes()
    assert lib.gspn_backward4_timed(1, 2, 8, 8, 2, 0, A, zs, ls, None, None, GY, DX, dzs, dls, None, WS, need, 0, 0,
                                    None, None) == NULLP
    assert lib.gspn_backward4_timed(1, 2, 8, 8, 2, 0, A, zs, ls, None, None, GY, DX, dzs, dls, None, WS, need - 1, 0,
                                    0, None, ctypes.byref(t)) == WSPACE


def test_layout_argument(lib):
    """GSPN_LAYOUT_ARRAY: the workspace grows by the scan-frame copies of the
    horizontal logits and lambdas (forward; twice that in the backward, for
    their gradients); an unknown layout is rejected before anything else,
    even for empty tensors; the array layout needs a workspace."""
    def copies(n, c, h, w, cw, es):
        return (2 * (3 * cw + c) * n * h * w * es + 3) // 4 * 4

    for (n, c, h, w, cw, dt) in [(1, 2, 8, 8, 2, 0), (1, 2, 8, 8, 1, 1), (2, 3, 6, 40, 3, 1), (1, 1, 3, 5, 1, 1)]:
        es = 4 if dt == 0 else 2
        base = lib.gspn_forward4_workspace_bytes(n, c, h, w, cw, dt, 0)
        assert lib.gspn_forward4_workspace_bytes(n, c, h, w, cw, dt, 1) == base + copies(n, c, h, w, cw, es)
        bb = lib.gspn_backward4_workspace_bytes(n, c, h, w, cw, dt, 0)
        assert lib.gspn_backward4_workspace_bytes(n, c, h, w, cw, dt, 1) == bb + 2 * copies(n, c, h, w, cw, es)
    assert lib.gspn_proxy_forward4_workspace_bytes(1, 6, 8, 8, 2, 1, 1, 1) == \
        2 * 2 * 64 * 2 + lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 1, 1, 1)
    for bad in (2, -1):
        assert lib.gspn_forward4_workspace_bytes(1, 2, 8, 8, 2, 0, bad) == -1
        assert lib.gspn_backward4_workspace_bytes(1, 2, 8, 8, 2, 0, bad) == -1
        assert lib.gspn_proxy_forward4_workspace_bytes(1, 6, 8, 8, 2, 1, 1, bad) == -1

    vp4 = ctypes.c_void_p * 4
    zs = vp4(B, B + 0x1000000, B + 0x2000000, B + 0x3000000)
    ls = vp4(C_, C_, C_, C_)
    W = 0x60000000
    need = lib.gspn_forward4_workspace_bytes(1, 2, 8, 80, 2, 0, 1)

    def f(n=1, lay=1, ws=W, wsb=need, x=A, y=D_):
        return lib.gspn_forward4(n, 2, 8, 80, 2, 0, x, zs, ls, None, y, None, ws, wsb, 0, lay, None)

    assert f(lay=2) == LAYOUT
    assert f(n=0, x=0, y=0, ws=0, wsb=0, lay=7) == LAYOUT   # enum checks run before the empty-tensor return
    assert f(ws=None, wsb=0) == WSPACE                      # the copies live in the workspace
    assert f(wsb=lib.gspn_forward4_workspace_bytes(1, 2, 8, 80, 2, 0, 0)) == WSPACE  # the scan layout's is too small
    assert f(ws=A + 16) == ALIAS
    assert f(n=0, x=0, y=0) == OK

    WD, WU, WS = 0x70000000, 0x71000000, 0x72000000
    pneed = lib.gspn_proxy_forward4_workspace_bytes(1, 6, 8, 8, 2, 1, 1, 1)
    assert lib.gspn_proxy_forward4(1, 6, 8, 8, 2, 1, 0, A, WD, WU, zs, ls, None, D_, None, WS, pneed, 1, 3,
                                   None) == LAYOUT
    assert lib.gspn_proxy_forward4(1, 6, 8, 8, 2, 1, 0, A, WD, WU, zs, ls, None, D_, None, WS, pneed - 1, 1, 1,
                                   None) == WSPACE

    dzs = vp4(0x40000000, 0x41000000, 0x42000000, 0x43000000)
    dls = vp4(0x44000000, 0x45000000, 0x46000000, 0x47000000)
    bneed = lib.gspn_backward4_workspace_bytes(1, 2, 8, 80, 2, 0, 1)

    def g(lay=1, wsb=bneed, s=None):
        return lib.gspn_backward4(1, 2, 8, 80, 2, 0, A, zs, ls, None, s, 0x50000000, 0x51000000, dzs, dls, None, WS,
                                  wsb, 0, lay, None)

    assert g(lay=-3) == LAYOUT
    assert g(wsb=bneed - 1) == WSPACE
    assert g(wsb=lib.gspn_backward4_workspace_bytes(1, 2, 8, 80, 2, 0, 0)) == WSPACE
    # with the states passed, the states' room (last) is not needed in either layout
    assert g(s=0x6a000000, wsb=bneed - 16 * 2 * 8 * 80 - 1) == WSPACE


def test_noalloc_validation(lib):
    """gspn_forward4_noalloc validates like gspn_forward4 and rejects calls
    whose workspace would exceed its static scratch before touching any
    device (nothing here reaches a device: there is none in this suite)."""
    vp4 = ctypes.c_void_p * 4
    zs = vp4(B, B + 0x1000000, B + 0x2000000, B + 0x3000000)
    ls = vp4(C_, C_, C_, C_)

    def f(n=1, c=2, h=8, w=80, cw=2, chunk=0, x=A, m=None, y=D_, s=None, dt=0, lay=0):
        return lib.gspn_forward4_noalloc(n, c, h, w, cw, chunk, x, zs, ls, m, y, s, dt, lay, None)

    assert f(dt=3) == DTYPE
    assert f(lay=4) == LAYOUT
    assert f(chunk=-1) == CHUNK
    assert f(x=0) == NULLP
    assert f(y=A) == ALIAS
    assert f(n=0, x=0, y=0) == OK
    assert G.NOALLOC_SCRATCH_BYTES == 64 << 20
    # 32 planes of 1024 x 1024 fp32: four maps alone are 512 MiB
    big = lib.gspn_forward4_workspace_bytes(32, 1, 1024, 1024, 1, 0, 0)
    assert big > G.NOALLOC_SCRATCH_BYTES
    assert f(n=32, c=1, h=1024, w=1024, cw=1) == WSPACE
    # the array layout's copies count against the scratch too
    small = (1, 4, 512, 1024, 4, 0)
    assert lib.gspn_forward4_workspace_bytes(*small, 0) <= G.NOALLOC_SCRATCH_BYTES
    assert lib.gspn_forward4_workspace_bytes(*small, 1) > G.NOALLOC_SCRATCH_BYTES
    assert f(n=1, c=4, h=512, w=1024, cw=4, lay=1) == WSPACE


def test_proxy_backward4_validation(lib):
    """gspn_proxy_backward4 rejects bad arguments before queueing anything
    (every call here fails validation)."""
    vp4 = ctypes.c_void_p * 4
    n, c, h, w, cp = 1, 6, 8, 8, 2
    es = 2
    zs = vp4(*[0x10000000 + d * 0x100000 for d in range(4)])
    ls = vp4(*[0x20000000 + d * 0x100000 for d in range(4)])
    dzs = vp4(*[0x30000000 + d * 0x100000 for d in range(4)])
    dls = vp4(*[0x40000000 + d * 0x100000 for d in range(4)])
    X, WD, WU, GY, DX, DWD, DWU, WS = (0x50000000, 0x51000000, 0x52000000, 0x53000000, 0x54000000, 0x55000000,
                                       0x56000000, 0x60000000)
    need = lib.gspn_proxy_backward4_workspace_bytes(n, c, h, w, cp, 1, 1, 0)
    assert need > 0 and need % 256 == 0
    assert lib.gspn_proxy_backward4_workspace_bytes(n, c, h, w, cp, 3, 1, 0) == -1     # cw neither 1 nor c_proxy
    assert lib.gspn_proxy_backward4_workspace_bytes(n, 0, h, w, cp, 1, 1, 0) == -1
    assert lib.gspn_proxy_backward4_workspace_bytes(n, c, h, w, 0, 1, 1, 0) == -1
    # at least the proxy-space backward's workspace
    assert need >= lib.gspn_backward4_workspace_bytes(n, cp, h, w, 1, 1, 0) + 4 * n * cp * h * w * es

    def f(n=n, c=c, h=h, w=w, cp=cp, cw=1, chunk=0, x=X, gy=GY, dx=DX, dwd=DWD, dwu=DWU, dz=dzs, dl=dls, m=None,
          dm=None, ws=WS, wsb=need, dt=1, lay=0, st=None):
        return lib.gspn_proxy_backward4(n, c, h, w, cp, cw, chunk, x, WD, WU, zs, ls, m, st, gy, dx, dwd, dwu, dz,
                                        dl, dm, ws, wsb, dt, lay, None)

    assert f(dt=2) == DTYPE
    assert f(lay=5) == LAYOUT
    assert f(c=0) == SHAPE
    assert f(cp=0) == SHAPE
    assert f(chunk=-1) == CHUNK
    assert f(cw=3) == WCH
    assert f(h=5000) == UNSUP
    assert f(x=0) == NULLP
    assert f(dwu=0) == NULLP
    assert f(dl=vp4(0x40000000, 0, 0x40200000, 0x40300000)) == NULLP
    assert f(ws=0) == NULLP
    assert f(wsb=need - 1) == WSPACE
    assert f(ws=WS + 2) == MISAL
    assert f(dx=DX + 1) == MISAL
    assert f(dwd=DWD + 2) == MISAL
    assert f(dx=X) == ALIAS                                   # dx over x
    assert f(dwu=DWD + 4) == ALIAS                            # the two weight gradients overlap
    assert f(dm=WS + 64, m=None) == ALIAS                     # dmerge inside the workspace
    assert f(dwd=WD) == ALIAS                                 # a gradient over its weights
    assert f(ws=GY - 64) == ALIAS                             # the workspace over gy
    assert f(h=3000, wsb=1 << 40) == UNSUP                    # longer lines than the proxy-space backward takes
    t = G.StageTimes()
    assert lib.gspn_proxy_backward4_timed(n, c, h, w, cp, 1, 0, X, WD, WU, zs, ls, None, None, GY, DX, DWD, DWU,
                                          dzs, dls, None, WS, need, 1, 0, None, None) == NULLP
    assert lib.gspn_proxy_backward4_timed(n, c, h, w, cp, 1, 0, X, WD, WU, zs, ls, None, None, GY, DX, DWD, DWU,
                                          dzs, dls, None, WS, need, 2, 0, None, ctypes.byref(t)) == DTYPE
    # kept proxy-space state: its size, alignment and aliasing
    kb = lib.gspn_proxy_states_bytes(n, cp, h, w, 1)
    pe = n * cp * h * w
    small = (h <= 64 and w <= 64)
    assert kb == 2 * ((pe * es + 255) // 256 * 256) + (0 if small else 16 * pe)
    assert lib.gspn_proxy_states_bytes(n, 0, h, w, 1) == -1 and lib.gspn_proxy_states_bytes(n, cp, h, w, 2) == -1
    ST = 0x7E000000
    assert f(st=ST + 16) == MISAL                             # 256-byte alignment
    assert f(st=WS + 256) == ALIAS                            # inside the workspace
    assert f(st=DX - 256) == ALIAS                            # over an output

