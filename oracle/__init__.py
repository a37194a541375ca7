"""fp64 CPU oracle for GSPN's 2D line-scan linear propagation.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product
path (the HIP library ``libgspn`` and its Python binding) never imports,
loads or calls anything here, and this package imports nothing from the
product package.

The arithmetic lives in ``gspn_oracle.c`` (plain loops, double precision,
OpenMP over independent planes); this module only marshals numpy arrays into
it.  Each wrapper cites the passage of the GSPN pages it follows; the C file
holds the full list of readings taken where the pages are silent.

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``,
``tests/test_oracle_backward_pins.py``, ``tests/test_oracle_merge_pins.py``
and ``tests/test_oracle_proxy_backward_pins.py`` (closed forms, brute-force
dense matrices, exact rational arithmetic, symmetry invariants, library
routines, and for the gradients central finite differences of the pinned
forward and adjoint dot-product and homogeneity identities); none is "parity
unpinned".

Layouts (contiguous, row-major):
  x, y, h           [N][C][H][W]
  logits, w (dir d) [N][Cw][3][S][L]   scan frame of direction d
  lam (dir d)       [N][C][S][L]       scan frame of direction d
Vertical directions (T2B, B2T): S = H, L = W (scan frame = array frame).
Horizontal directions (L2R, R2L): S = W, L = H (step i = column i, line
position k = row k), i.e. the transpose of the array frame.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import sys
import threading
from typing import Sequence

import numpy as np

DIRECTIONS = ("T2B", "B2T", "L2R", "R2L")
T2B, B2T, L2R, R2L = 0, 1, 2, 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gspn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_handle = None


def build(force: bool = False) -> str:
    """Compile ``gspn_oracle.c`` into ``liboracle.so`` with gcc (plain C,
    OpenMP, no FMA contraction so every product is rounded as written)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _lib():
    global _handle
    with _lock:
        if _handle is None:
            build()
            lib = ctypes.CDLL(_LIB)
            i64 = ctypes.c_int64
            dp = ctypes.POINTER(ctypes.c_double)
            lib.oracle_normalize.argtypes = [ctypes.c_int, i64, i64, i64, i64, dp, dp]
            lib.oracle_scan.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, dp, dp,
                                        ctypes.c_int, dp, dp, ctypes.c_int]
            lib.oracle_forward4.argtypes = [i64, i64, i64, i64, i64, i64, dp,
                                            ctypes.POINTER(dp), ctypes.POINTER(dp), dp]
            lib.oracle_project.argtypes = [i64, i64, i64, i64, dp, dp, dp]
            for f in (lib.oracle_normalize, lib.oracle_scan, lib.oracle_forward4,
                      lib.oracle_project):
                f.restype = ctypes.c_int
            lib.oracle_scan_backward.argtypes = [ctypes.c_int, i64, i64, i64, i64, i64, i64, dp, dp, dp, dp,
                                                 dp, dp, dp]
            lib.oracle_scan_backward.restype = ctypes.c_int
            lib.oracle_backward4.argtypes = [i64, i64, i64, i64, i64, i64, dp, ctypes.POINTER(dp),
                                             ctypes.POINTER(dp), dp, dp, ctypes.POINTER(dp), ctypes.POINTER(dp)]
            lib.oracle_backward4.restype = ctypes.c_int
            lib.oracle_max_threads.argtypes = []
            lib.oracle_max_threads.restype = ctypes.c_int
            _handle = lib
        return _handle


def _f64(a) -> np.ndarray:
    """Contiguous float64 copy/view of a numpy array or a CPU torch tensor
    (bf16 and fp32 values widen to fp64 exactly)."""
    if hasattr(a, "detach"):  # torch tensor, converted without importing torch here
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def frame_shape(direction: int, h: int, w: int) -> tuple[int, int]:
    """(S, L) = (number of scan steps, line length) of a direction."""
    return (w, h) if direction in (L2R, R2L) else (h, w)


def _array_hw(direction: int, S: int, L: int) -> tuple[int, int]:
    return (L, S) if direction in (L2R, R2L) else (S, L)


def normalize(direction: int, logits) -> np.ndarray:
    """Sigmoid + row normalisation of the three neighbour logits
    (GSPN summary page, "Approach"; GSPN-2 notes, "2D spatial propagation
    recap": tridiagonal, rows sum to 1).  logits [N][Cw][3][S][L] -> w."""
    z = _f64(logits)
    n, cw, three, S, L = z.shape
    assert three == 3
    h, w = _array_hw(direction, S, L)
    out = np.empty_like(z)
    rc = _lib().oracle_normalize(direction, n, cw, h, w, _ptr(z), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_normalize rejected its arguments")
    return out


def scan(direction: int, x, wts, lam, chunk: int = 0, wts_are_logits: bool = True,
         out: np.ndarray | None = None, accumulate: bool = False) -> np.ndarray:
    """One direction of the line scan h_i = w_i h_{i-1} + lam_i * x_i
    (GSPN-2 notes, "2D spatial propagation recap"), optionally cut into
    independent chunks of ``chunk`` steps (GSPN-2 notes, "Optimisation 1").
    x [N][C][H][W]; wts [N][Cw][3][S][L] (Cw = 1 or C); lam [N][C][S][L]."""
    xx = _f64(x)
    n, c, h, w = xx.shape
    S, L = frame_shape(direction, h, w)
    ww = _f64(wts)
    ll = _f64(lam)
    if ww.shape[0] != n or ww.shape[2:] != (3, S, L) or ww.shape[1] not in (1, c):
        raise ValueError("wts shape %r does not fit x %r for direction %s"
                         % (ww.shape, xx.shape, DIRECTIONS[direction]))
    if ll.shape != (n, c, S, L):
        raise ValueError("lam shape %r does not fit x %r" % (ll.shape, xx.shape))
    if out is None:
        out = np.zeros((n, c, h, w), dtype=np.float64)
        accumulate = False
    assert out.dtype == np.float64 and out.flags.c_contiguous and out.shape == (n, c, h, w)
    rc = _lib().oracle_scan(direction, int(chunk), n, c, h, w, ww.shape[1], _ptr(xx), _ptr(ww),
                            1 if wts_are_logits else 0, _ptr(ll), _ptr(out),
                            1 if accumulate else 0)
    if rc != 0:
        raise ValueError("oracle_scan rejected its arguments")
    return out


def _merge_weights(merge, c: int) -> np.ndarray:
    m = _f64(merge)
    if m.shape != (4, c):
        raise ValueError("merge weights %r do not fit (4, %d)" % (m.shape, c))
    return m


def forward4(x, logits: Sequence, lams: Sequence, chunk: int = 0, merge=None) -> np.ndarray:
    """All four directions on the same x (four line scans, GSPN-2 notes, "2D
    spatial propagation recap"), merged by an elementwise sum, or with
    ``merge`` [4][C] by the learnable merge that the GSPN summary page's
    ablation table puts in place of max-pooling, read as one weight per
    direction and channel: y[:, c] = sum_d merge[d, c] h_d[:, c]."""
    xx = _f64(x)
    n, c, h, w = xx.shape
    if merge is not None:
        m = _merge_weights(merge, c)
        y = np.zeros((n, c, h, w), dtype=np.float64)
        for d in range(4):
            y += m[d][None, :, None, None] * scan(d, xx, logits[d], lams[d], chunk)
        return y
    zs = [_f64(z) for z in logits]
    ls = [_f64(l) for l in lams]
    cw = zs[0].shape[1]
    for d in range(4):
        S, L = frame_shape(d, h, w)
        if zs[d].shape != (n, cw, 3, S, L) or ls[d].shape != (n, c, S, L):
            raise ValueError("direction %s tensors do not fit x" % DIRECTIONS[d])
    y = np.empty((n, c, h, w), dtype=np.float64)
    zp = (ctypes.POINTER(ctypes.c_double) * 4)(*[_ptr(z) for z in zs])
    lp = (ctypes.POINTER(ctypes.c_double) * 4)(*[_ptr(l) for l in ls])
    rc = _lib().oracle_forward4(n, c, h, w, cw, int(chunk), _ptr(xx), zp, lp, _ptr(y))
    if rc != 0:
        raise ValueError("oracle_forward4 rejected its arguments")
    return y


def project(inp, weight) -> np.ndarray:
    """1x1 projection between channel spaces, out[n,o] = sum_c W[o,c] in[n,c]
    (GSPN-2 notes, "Optimisation 2", compressive channel proxy).  No bias."""
    a = _f64(inp)
    wt = _f64(weight)
    n, cin, h, w = a.shape
    cout, cin2 = wt.shape
    if cin2 != cin:
        raise ValueError("weight %r does not fit input channels %d" % (wt.shape, cin))
    out = np.empty((n, cout, h, w), dtype=np.float64)
    rc = _lib().oracle_project(n, cin, h * w, cout, _ptr(a), _ptr(wt), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_project rejected its arguments")
    return out


def proxy_forward4(x, w_down, w_up, logits: Sequence, lams: Sequence, chunk: int = 0, merge=None) -> np.ndarray:
    """Compressive-proxy forward: project C -> C_proxy, run the four-direction
    scan in proxy space (merge weights, if any, over the proxy channels),
    project back C_proxy -> C (GSPN-2 notes, "Optimisation 2")."""
    xp = project(x, w_down)
    yp = forward4(xp, logits, lams, chunk, merge=merge)
    return project(yp, w_up)


def scan_backward(direction: int, x, logits, lam, gy, chunk: int = 0):
    """Gradient of one direction's scan (the exact derivative of ``scan``):
    returns (dx, dlam, dlogits) for dL/dh = gy.  x, gy [N][C][H][W];
    logits [N][Cw][3][S][L]; lam [N][C][S][L].  Channel-shared logits get
    the sum over channels."""
    xx = _f64(x)
    n, c, h, w = xx.shape
    S, L = frame_shape(direction, h, w)
    zz = _f64(logits)
    ll = _f64(lam)
    gg = _f64(gy)
    cw = zz.shape[1]
    if zz.shape != (n, cw, 3, S, L) or ll.shape != (n, c, S, L) or gg.shape != xx.shape:
        raise ValueError("shapes do not fit x for direction %s" % DIRECTIONS[direction])
    dx = np.zeros_like(xx)
    dl = np.empty_like(ll)
    dz = np.zeros_like(zz)
    rc = _lib().oracle_scan_backward(direction, int(chunk), n, c, h, w, cw, _ptr(xx), _ptr(zz), _ptr(ll),
                                     _ptr(gg), _ptr(dx), _ptr(dl), _ptr(dz))
    if rc != 0:
        raise ValueError("oracle_scan_backward rejected its arguments")
    return dx, dl, dz


def backward4(x, logits: Sequence, lams: Sequence, gy, chunk: int = 0, merge=None):
    """Gradient of forward4 for dL/dy = gy: (dx, [dlam_d], [dlogits_d]), and
    with ``merge`` also dmerge [4][C].  With merge weights m, direction d's
    output enters y as m[d, c] h_d, so its scan receives dL/dh_d =
    m[d, c] gy, and dL/dm[d, c] = sum over images and positions of
    gy * h_d (h_d recomputed by ``scan``)."""
    xx = _f64(x)
    n, c, h, w = xx.shape
    zs = [_f64(z) for z in logits]
    ls = [_f64(l) for l in lams]
    gg = _f64(gy)
    cw = zs[0].shape[1]
    if merge is not None:
        m = _merge_weights(merge, c)
        if gg.shape != xx.shape:
            raise ValueError("gy does not fit x")
        dx = np.zeros_like(xx)
        dls, dzs = [], []
        dm = np.zeros((4, c), dtype=np.float64)
        for d in range(4):
            dxd, dld, dzd = scan_backward(d, xx, zs[d], ls[d], m[d][None, :, None, None] * gg, chunk)
            dx += dxd
            dls.append(dld)
            dzs.append(dzd)
            dm[d] = np.sum(gg * scan(d, xx, zs[d], ls[d], chunk), axis=(0, 2, 3))
        return dx, dls, dzs, dm
    for d in range(4):
        S, L = frame_shape(d, h, w)
        if zs[d].shape != (n, cw, 3, S, L) or ls[d].shape != (n, c, S, L):
            raise ValueError("direction %s tensors do not fit x" % DIRECTIONS[d])
    if gg.shape != xx.shape:
        raise ValueError("gy does not fit x")
    dx = np.empty_like(xx)
    dls = [np.empty_like(l) for l in ls]
    dzs = [np.empty_like(z) for z in zs]
    dp = ctypes.POINTER(ctypes.c_double)
    rc = _lib().oracle_backward4(n, c, h, w, cw, int(chunk), _ptr(xx), (dp * 4)(*[_ptr(z) for z in zs]),
                                 (dp * 4)(*[_ptr(l) for l in ls]), _ptr(gg), _ptr(dx),
                                 (dp * 4)(*[_ptr(a) for a in dls]), (dp * 4)(*[_ptr(a) for a in dzs]))
    if rc != 0:
        raise ValueError("oracle_backward4 rejected its arguments")
    return dx, dls, dzs


def proxy_backward4(x, w_down, w_up, logits: Sequence, lams: Sequence, gy, chunk: int = 0, merge=None):
    """Gradient of proxy_forward4 for dL/dy = gy, by the chain rule through
    its three stages (GSPN-2 notes, "Optimisation 2": x_p = W_down x,
    y_p = forward4(x_p), y = W_up y_p, all 1x1 projections without bias):
      dL/dy_p  = W_up^T gy                  (a projection with W_up^T)
      dx_p, dlam_d, dlogits_d (, dmerge) = backward4 in proxy space for dL/dy_p
      dx       = W_down^T dx_p               (a projection with W_down^T)
      dW_up[c][k]   = sum over images and pixels of gy[c] * y_p[k]
      dW_down[k][c] = sum over images and pixels of dx_p[k] * x[c]
    Returns (dx, dW_down [C_proxy][C], dW_up [C][C_proxy], [dlam_d],
    [dlogits_d]) and, with ``merge``, dmerge [4][C_proxy] last."""
    xx = _f64(x)
    wd = _f64(w_down)
    wu = _f64(w_up)
    gg = _f64(gy)
    if gg.shape != xx.shape:
        raise ValueError("gy does not fit x")
    xp = project(xx, wd)
    yp = forward4(xp, logits, lams, chunk, merge=merge)
    gp = project(gg, wu.T)
    res = backward4(xp, logits, lams, gp, chunk, merge=merge)
    dxp = res[0]
    dx = project(dxp, wd.T)
    n = xx.shape[0]
    dwu = sum(gg[i].reshape(gg.shape[1], -1) @ yp[i].reshape(yp.shape[1], -1).T for i in range(n))
    dwd = sum(dxp[i].reshape(dxp.shape[1], -1) @ xx[i].reshape(xx.shape[1], -1).T for i in range(n))
    out = (dx, dwd, dwu, res[1], res[2])
    return out + (res[3],) if merge is not None else out


def max_threads() -> int:
    """Threads the oracle's OpenMP loops may use (OMP_NUM_THREADS, else all
    cores)."""
    return int(_lib().oracle_max_threads())


def normwise_error(got, ref) -> float:
    """max_i |got_i - ref_i| / max_i |ref_i| (0 when both are all zero)."""
    g = _f64(got)
    r = _f64(ref)
    den = float(np.max(np.abs(r))) if r.size else 0.0
    num = float(np.max(np.abs(g - r))) if r.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


if __name__ == "__main__":  # pragma: no cover
    print(build(force="--force" in sys.argv))
