"""Pins of the oracle's backward pass (CPU only).

The gradient is the exact derivative of the forward propagation, which the
oracle's forward already implements and ``test_oracle_pins.py`` pins.  These
tests tie the backward to things independent of its adjoint derivation:
  - central finite differences of <gy, forward4(x, logits, lam)> in fp64, for
    every element of dx, dlam and dlogits (per-channel and shared logits,
    full and chunked scans, square and rectangular planes);
  - the exact adjoint identities <dx, x> = <gy, y> and sum_d <dlam_d, lam_d> =
    <gy, y> (y is linear in x and in each lam_d);
  - closed forms: a line of length 1 has w = [1] whatever its logits, so their
    gradient is 0; with chunk length 1 every step starts a chunk, so dlogits =
    0, dlam_d = gy * x and dx = sum_d gy * lam_d; the logits of each chunk's
    first line are unused, so their gradient is 0;
  - shared logits receive the sum over channels of the per-channel gradient;
  - reversing the scan axis of every input reverses the gradients.
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
    gy = rng.standard_normal((n, c, h, w))
    return x, zs, ls, gy


def _loss(x, zs, ls, gy, chunk):
    return float(np.sum(gy * oracle.forward4(x, zs, ls, chunk=chunk)))


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
    scale = 1.0 + max(float(np.max(np.abs(a))), float(np.max(np.abs(b))))
    assert np.max(np.abs(a - b)) <= tol * scale, np.max(np.abs(a - b))


@pytest.mark.parametrize("n,c,h,w,shared,chunk", [
    (1, 2, 4, 5, False, 0),
    (1, 2, 5, 4, False, 2),
    (2, 1, 3, 6, False, 4),
    (1, 3, 4, 4, True, 0),
    (1, 2, 5, 3, True, 3),
])
def test_gradients_match_finite_differences(n, c, h, w, shared, chunk):
    rng = np.random.default_rng(1000 + 7 * h + w + chunk)
    x, zs, ls, gy = _inputs(rng, n, c, h, w, 1 if shared else c)
    dx, dls, dzs = oracle.backward4(x, zs, ls, gy, chunk=chunk)
    f = lambda: _loss(x, zs, ls, gy, chunk)
    _close(dx, _fd(x, f))
    for d in range(4):
        _close(dls[d], _fd(ls[d], f))
        _close(dzs[d], _fd(zs[d], f))


@pytest.mark.parametrize("chunk", [0, 3])
def test_adjoint_dot_product_identities(chunk):
    rng = np.random.default_rng(77)
    x, zs, ls, gy = _inputs(rng, 2, 3, 9, 11, 3)
    y = oracle.forward4(x, zs, ls, chunk=chunk)
    dx, dls, _ = oracle.backward4(x, zs, ls, gy, chunk=chunk)
    ref = float(np.sum(gy * y))
    assert abs(float(np.sum(dx * x)) - ref) <= 1e-11 * (1 + abs(ref))
    assert abs(sum(float(np.sum(dls[d] * ls[d])) for d in range(4)) - ref) <= 1e-11 * (1 + abs(ref))


def test_single_direction_gradient_sums_to_backward4():
    rng = np.random.default_rng(5)
    x, zs, ls, gy = _inputs(rng, 1, 2, 6, 7, 2)
    dx, dls, dzs = oracle.backward4(x, zs, ls, gy, chunk=4)
    acc = np.zeros_like(x)
    for d in range(4):
        dxd, dld, dzd = oracle.scan_backward(d, x, zs[d], ls[d], gy, chunk=4)
        acc += dxd
        np.testing.assert_array_equal(dld, dls[d])
        np.testing.assert_array_equal(dzd, dzs[d])
    np.testing.assert_allclose(acc, dx, rtol=0, atol=1e-13)


def test_length_one_lines_have_no_logit_gradient():
    rng = np.random.default_rng(6)
    # H = 1: horizontal lines (columns) have length 1, vertical scans a single step
    x, zs, ls, gy = _inputs(rng, 1, 2, 1, 7, 2)
    _, _, dzs = oracle.backward4(x, zs, ls, gy)
    assert all(np.all(dz == 0) for dz in dzs)
    # W = 1: vertical lines (rows) have length 1
    x, zs, ls, gy = _inputs(rng, 1, 2, 7, 1, 2)
    _, _, dzs = oracle.backward4(x, zs, ls, gy)
    assert np.all(dzs[0] == 0) and np.all(dzs[1] == 0)


def test_chunk_one_closed_form():
    rng = np.random.default_rng(8)
    n, c, h, w = 1, 2, 5, 6
    x, zs, ls, gy = _inputs(rng, n, c, h, w, c)
    dx, dls, dzs = oracle.backward4(x, zs, ls, gy, chunk=1)
    expect_dx = np.zeros_like(x)
    for d in range(4):
        assert np.all(dzs[d] == 0)
        lam_arr = ls[d] if d < 2 else np.swapaxes(ls[d], 2, 3)   # into the array frame
        dl_arr = dls[d] if d < 2 else np.swapaxes(dls[d], 2, 3)
        np.testing.assert_allclose(dl_arr, gy * x, rtol=0, atol=1e-15)
        expect_dx += gy * lam_arr
    np.testing.assert_allclose(dx, expect_dx, rtol=0, atol=1e-14)


@pytest.mark.parametrize("chunk", [0, 3])
def test_first_line_of_each_chunk_has_no_logit_gradient(chunk):
    rng = np.random.default_rng(9)
    n, c, h, w = 1, 2, 7, 6
    x, zs, ls, gy = _inputs(rng, n, c, h, w, c)
    _, _, dzs = oracle.backward4(x, zs, ls, gy, chunk=chunk)
    for d in range(4):
        S, _ = frame_shape(d, h, w)
        K = S if chunk == 0 else chunk
        rev = d in (1, 3)
        for t in range(S):
            i = S - 1 - t if rev else t
            if t % K == 0:
                assert np.all(dzs[d][:, :, :, i, :] == 0), (d, t)
            else:
                assert np.any(dzs[d][:, :, :, i, :] != 0), (d, t)


def test_shared_logits_receive_the_channel_sum():
    rng = np.random.default_rng(10)
    n, c, h, w = 2, 3, 5, 4
    x, zs, ls, gy = _inputs(rng, n, c, h, w, 1)
    _, _, dz_shared = oracle.backward4(x, zs, ls, gy, chunk=2)
    zb = [np.ascontiguousarray(np.broadcast_to(z, (n, c) + z.shape[2:])) for z in zs]
    _, _, dz_each = oracle.backward4(x, zb, ls, gy, chunk=2)
    for d in range(4):
        np.testing.assert_allclose(dz_shared[d], dz_each[d].sum(axis=1, keepdims=True), rtol=1e-12, atol=1e-14)


def test_reversal_flips_the_gradients():
    """B2T on inputs flipped along H equals T2B flipped back (R2L / L2R along
    W).  In the scan frame the flip is along S: logits axis 3, lam axis 2."""
    rng = np.random.default_rng(11)
    n, c, h, w = 1, 2, 6, 5
    x, zs, ls, gy = _inputs(rng, n, c, h, w, c)
    for fwd, rev, arr_axis in ((0, 1, 2), (2, 3, 3)):
        dx_f, dl_f, dz_f = oracle.scan_backward(fwd, x, zs[fwd], ls[fwd], gy, chunk=4)
        dx_r, dl_r, dz_r = oracle.scan_backward(rev, np.flip(x, arr_axis).copy(), np.flip(zs[fwd], 3).copy(),
                                                np.flip(ls[fwd], 2).copy(), np.flip(gy, arr_axis).copy(),
                                                chunk=4)
        np.testing.assert_allclose(np.flip(dx_r, arr_axis), dx_f, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(np.flip(dl_r, 2), dl_f, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(np.flip(dz_r, 3), dz_f, rtol=1e-12, atol=1e-13)
