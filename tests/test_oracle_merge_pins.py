"""Pins of the oracle's learnable merge (CPU only).

The merge weights m [4][C] enter as y[:, c] = sum_d m[d, c] h_d[:, c] (the
learnable merging of the GSPN summary page's ablation table, read as one
weight per direction and channel).  These tests tie it to facts that do not
depend on the merge code:
  - m = 1 everywhere is the plain sum, and a one-hot m over directions picks
    that direction's scan alone;
  - the closed form for constant input: with lambda = 1 and x = v, direction
    d's state at scan step t is (t + 1) v whatever the logits, so
    y[i, j] = v (m_T2B (i + 1) + m_B2T (H - i) + m_L2R (j + 1) + m_R2L (W - j))
    per channel; a swapped direction or channel index fails it;
  - y is linear in m;
  - central finite differences of <gy, y> for dm, dx, dlam and dlogits;
  - the exact identity sum_{d,c} m[d, c] dm[d, c] = <gy, y> (y is linear in m).
"""
import numpy as np
import pytest

import oracle
from oracle import frame_shape

pytestmark = pytest.mark.filterwarnings("ignore")


def _inputs(rng, n, c, h, w, cw):
    x = rng.standard_normal((n, c, h, w))
    zs, ls = [], []
    for d in range(4):
        S, L = frame_shape(d, h, w)
        zs.append(rng.standard_normal((n, cw, 3, S, L)))
        ls.append(rng.random((n, c, S, L)))
    return x, zs, ls


def test_unit_merge_is_the_sum():
    rng = np.random.default_rng(1)
    x, zs, ls = _inputs(rng, 2, 3, 7, 9, 3)
    y0 = oracle.forward4(x, zs, ls, chunk=4)
    y1 = oracle.forward4(x, zs, ls, chunk=4, merge=np.ones((4, 3)))
    np.testing.assert_allclose(y1, y0, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("d", [0, 1, 2, 3])
def test_one_hot_merge_selects_a_direction(d):
    rng = np.random.default_rng(2 + d)
    x, zs, ls = _inputs(rng, 1, 2, 6, 5, 1)
    m = np.zeros((4, 2))
    m[d] = 1.0
    y = oracle.forward4(x, zs, ls, merge=m)
    np.testing.assert_allclose(y, oracle.scan(d, x, zs[d], ls[d]), rtol=0, atol=0)


def test_constant_input_closed_form():
    rng = np.random.default_rng(3)
    n, c, h, w = 2, 3, 6, 9
    _, zs, _ = _inputs(rng, n, c, h, w, c)
    x = np.full((n, c, h, w), 0.5)
    ls = [np.ones((n, c) + frame_shape(d, h, w)) for d in range(4)]
    m = rng.standard_normal((4, c))
    y = oracle.forward4(x, zs, ls, merge=m)
    i = np.arange(h)[:, None]
    j = np.arange(w)[None, :]
    for ch in range(c):
        expect = 0.5 * (m[0, ch] * (i + 1) + m[1, ch] * (h - i) + m[2, ch] * (j + 1) + m[3, ch] * (w - j))
        for b in range(n):
            np.testing.assert_allclose(y[b, ch], expect, rtol=1e-12, atol=1e-12)


def test_linear_in_the_merge_weights():
    rng = np.random.default_rng(4)
    x, zs, ls = _inputs(rng, 1, 2, 5, 7, 2)
    m1, m2 = rng.standard_normal((4, 2)), rng.standard_normal((4, 2))
    y = oracle.forward4(x, zs, ls, chunk=3, merge=m1 + 2.0 * m2)
    y1 = oracle.forward4(x, zs, ls, chunk=3, merge=m1)
    y2 = oracle.forward4(x, zs, ls, chunk=3, merge=m2)
    np.testing.assert_allclose(y, y1 + 2.0 * y2, rtol=1e-12, atol=1e-12)


def _fd(arr, f, eps=1e-5):
    g = np.empty_like(arr)
    flat, gf = arr.reshape(-1), g.reshape(-1)
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
    scale = 1.0 + max(float(np.max(np.abs(a))), float(np.max(np.abs(b))))
    assert np.max(np.abs(a - b)) <= tol * scale, np.max(np.abs(a - b))


@pytest.mark.parametrize("n,c,h,w,shared,chunk", [
    (1, 2, 4, 5, False, 0),
    (1, 3, 5, 4, True, 2),
])
def test_merge_gradients_match_finite_differences(n, c, h, w, shared, chunk):
    rng = np.random.default_rng(50 + h * w + chunk)
    x, zs, ls = _inputs(rng, n, c, h, w, 1 if shared else c)
    gy = rng.standard_normal(x.shape)
    m = rng.standard_normal((4, c))
    dx, dls, dzs, dm = oracle.backward4(x, zs, ls, gy, chunk=chunk, merge=m)
    f = lambda: float(np.sum(gy * oracle.forward4(x, zs, ls, chunk=chunk, merge=m)))
    _close(dm, _fd(m, f))
    _close(dx, _fd(x, f))
    for d in range(4):
        _close(dls[d], _fd(ls[d], f))
        _close(dzs[d], _fd(zs[d], f))


@pytest.mark.parametrize("chunk", [0, 3])
def test_merge_gradient_identity(chunk):
    rng = np.random.default_rng(60 + chunk)
    x, zs, ls = _inputs(rng, 2, 3, 8, 6, 3)
    gy = rng.standard_normal(x.shape)
    m = rng.standard_normal((4, 3))
    y = oracle.forward4(x, zs, ls, chunk=chunk, merge=m)
    _, dls, _, dm = oracle.backward4(x, zs, ls, gy, chunk=chunk, merge=m)
    ref = float(np.sum(gy * y))
    assert abs(float(np.sum(m * dm)) - ref) <= 1e-11 * (1 + abs(ref))
    # y is linear in each lam_d too, merged or not
    assert abs(sum(float(np.sum(dls[d] * ls[d])) for d in range(4)) - ref) <= 1e-11 * (1 + abs(ref))
