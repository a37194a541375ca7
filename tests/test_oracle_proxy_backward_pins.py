"""Pins of the oracle's compressive-proxy backward (CPU only).

``oracle.proxy_backward4`` chains the pinned projection, forward and backward
(GSPN-2 notes, "Optimisation 2").  It is tied here to things that do not
reuse its chain-rule derivation:
  - central finite differences of <gy, proxy_forward4(...)> in fp64 for every
    element of dx, dW_down, dW_up, dlam_d, dlogits_d and dmerge (per-channel
    and shared logits, full and chunked scans, with and without merge);
  - exact homogeneity identities: y is linear in x, in W_down, in W_up, in
    the lam maps together and in the merge weights, so <gy, y> equals
    <dx, x>, <dW_down, W_down>, <dW_up, W_up>, sum_d <dlam_d, lam_d> and
    <dmerge, merge>;
  - W_up = 0 leaves dL/dy_p = 0: every gradient but dW_up vanishes, and
    dW_up is then the plain sum of gy times the proxy output;
  - C_proxy = C with identity projections gives backward4's gradients.
"""
import numpy as np
import pytest

import oracle
from oracle import frame_shape

pytestmark = pytest.mark.filterwarnings("ignore")


def _inputs(rng, n, c, cp, h, w, shared):
    x = rng.standard_normal((n, c, h, w))
    wd = rng.standard_normal((cp, c)) / np.sqrt(c)
    wu = rng.standard_normal((c, cp)) / np.sqrt(cp)
    zs, ls = [], []
    for d in range(4):
        S, L = frame_shape(d, h, w)
        zs.append(rng.standard_normal((n, 1 if shared else cp, 3, S, L)))
        ls.append(rng.random((n, cp, S, L)))
    gy = rng.standard_normal((n, c, h, w))
    return x, wd, wu, zs, ls, gy


def _fd(arr, f, eps=1e-5):
    """Central differences of f() with respect to every element of arr (in place)."""
    g = np.empty_like(arr)
    flat = arr.reshape(-1)
    gf = g.reshape(-1)
    for e in range(flat.size):
        v = flat[e]
        flat[e] = v + eps
        fp = f()
        flat[e] = v - eps
        fm = f()
        flat[e] = v
        gf[e] = (fp - fm) / (2 * eps)
    return g


def _close(a, b, tol=2e-7):
    assert a.shape == b.shape, (a.shape, b.shape)
    scale = 1.0 + max(float(np.max(np.abs(a))), float(np.max(np.abs(b))))
    assert np.max(np.abs(a - b)) <= tol * scale, np.max(np.abs(a - b))


@pytest.mark.parametrize("n,c,cp,h,w,shared,chunk,merge", [
    (1, 3, 2, 4, 5, False, 0, False),
    (1, 4, 2, 5, 4, True, 2, False),
    (2, 3, 1, 3, 4, False, 3, True),
    (1, 2, 3, 4, 3, True, 0, True),
])
def test_gradients_match_finite_differences(n, c, cp, h, w, shared, chunk, merge):
    rng = np.random.default_rng(2000 + 11 * c + 5 * cp + h + chunk)
    x, wd, wu, zs, ls, gy = _inputs(rng, n, c, cp, h, w, shared)
    m = rng.standard_normal((4, cp)) if merge else None
    res = oracle.proxy_backward4(x, wd, wu, zs, ls, gy, chunk=chunk, merge=m)
    dx, dwd, dwu, dls, dzs = res[:5]
    f = lambda: float(np.sum(gy * oracle.proxy_forward4(x, wd, wu, zs, ls, chunk=chunk, merge=m)))
    _close(dx, _fd(x, f))
    _close(dwd, _fd(wd, f))
    _close(dwu, _fd(wu, f))
    for d in range(4):
        _close(dls[d], _fd(ls[d], f))
        _close(dzs[d], _fd(zs[d], f))
    if merge:
        _close(res[5], _fd(m, f))


@pytest.mark.parametrize("chunk,merge", [(0, False), (4, True)])
def test_homogeneity_identities(chunk, merge):
    rng = np.random.default_rng(2100 + chunk)
    x, wd, wu, zs, ls, gy = _inputs(rng, 2, 5, 3, 9, 11, False)
    m = rng.standard_normal((4, 3)) if merge else None
    y = oracle.proxy_forward4(x, wd, wu, zs, ls, chunk=chunk, merge=m)
    res = oracle.proxy_backward4(x, wd, wu, zs, ls, gy, chunk=chunk, merge=m)
    dx, dwd, dwu, dls, _ = res[:5]
    ref = float(np.sum(gy * y))
    tol = 1e-11 * (1 + abs(ref))
    assert abs(float(np.sum(dx * x)) - ref) <= tol
    assert abs(float(np.sum(dwd * wd)) - ref) <= tol
    assert abs(float(np.sum(dwu * wu)) - ref) <= tol
    assert abs(sum(float(np.sum(dls[d] * ls[d])) for d in range(4)) - ref) <= tol
    if merge:
        assert abs(float(np.sum(res[5] * m)) - ref) <= tol


def test_zero_up_projection():
    rng = np.random.default_rng(2200)
    x, wd, wu, zs, ls, gy = _inputs(rng, 1, 4, 2, 6, 5, False)
    wu = np.zeros_like(wu)
    dx, dwd, dwu, dls, dzs = oracle.proxy_backward4(x, wd, wu, zs, ls, gy, chunk=0)
    assert np.all(dx == 0) and np.all(dwd == 0)
    assert all(np.all(a == 0) for a in dls) and all(np.all(a == 0) for a in dzs)
    # dW_up[c][k] = sum over pixels of gy[c] * y_p[k], with y_p from the proxy forward
    yp = oracle.proxy_forward4(x, wd, np.eye(2), zs, ls, chunk=0)     # W_up = I exposes y_p
    for c in range(4):
        for k in range(2):
            assert abs(dwu[c, k] - float(np.sum(gy[:, c] * yp[:, k]))) <= 1e-12 * (1 + abs(dwu[c, k]))


def test_identity_projections_give_backward4():
    rng = np.random.default_rng(2300)
    c = 3
    x, _, _, zs, ls, gy = _inputs(rng, 1, c, c, 5, 6, True)
    eye = np.eye(c)
    dx, _, _, dls, dzs = oracle.proxy_backward4(x, eye, eye, zs, ls, gy, chunk=2)
    rx, rls, rzs = oracle.backward4(x, zs, ls, gy, chunk=2)
    np.testing.assert_allclose(dx, rx, rtol=0, atol=1e-13)
    for d in range(4):
        np.testing.assert_allclose(dls[d], rls[d], rtol=0, atol=1e-13)
        np.testing.assert_allclose(dzs[d], rzs[d], rtol=0, atol=1e-13)
