"""Pins for the fp64 CPU oracle against what the GSPN pages and mathematics fix.

Each test checks the oracle against something other than itself: exact values
worked out from the definition by hand, closed forms, an independent dense
block-lower-triangular construction of the unrolled scan (H = G X, GSPN-2
notes, "Optimisation 2", linear-attention reading), exact rational
arithmetic, library routines (numpy cumsum / einsum) and symmetry invariants.
The pages print no worked numerical example, so these are the pins.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
from oracle import T2B, B2T, L2R, R2L

rng = np.random.default_rng(1234)


def _frame(direction, h, w):
    return oracle.frame_shape(direction, h, w)


def _rand_logits(n, cw, S, L, scale=1.0):
    return rng.normal(0.0, scale, size=(n, cw, 3, S, L))


# ----------------------------------------------------------------------------
# Normalisation (sigmoid + row normalisation; rows sum to 1)
# ----------------------------------------------------------------------------

def test_normalize_rows_sum_to_one_and_borders_are_zero():
    z = _rand_logits(2, 3, 7, 9, scale=4.0)
    z[0, 0, :, 0, 0] = [-700.0, 30.0, -30.0]   # extreme but finite logits
    w = oracle.normalize(T2B, z)
    s = w.sum(axis=2)
    assert np.max(np.abs(s - 1.0)) < 1e-15
    assert np.all(w[:, :, 0, :, 0] == 0.0)        # no left neighbour at k = 0
    assert np.all(w[:, :, 2, :, -1] == 0.0)       # no right neighbour at k = L-1
    inner = w[:, :, :, :, 1:-1]
    assert np.all(inner > 0.0) and np.all(inner < 1.0)


def test_normalize_zero_logits_gives_uniform_rows():
    # sigmoid(0) = 1/2 everywhere: interior rows 1/3 each, border rows 1/2 each.
    w = oracle.normalize(T2B, np.zeros((1, 1, 3, 4, 5)))
    assert np.all(w[0, 0, :, :, 1:4] == pytest.approx(1.0 / 3.0, abs=1e-16))
    assert np.all(w[0, 0, 1:, :, 0] == pytest.approx(0.5, abs=1e-16))
    assert np.all(w[0, 0, :2, :, 4] == pytest.approx(0.5, abs=1e-16))


def test_normalize_hand_worked_values():
    # sigmoid(-ln 3) = 1/4, sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4; their sum is 3/2.
    ln3 = math.log(3.0)
    L = 3
    z = np.zeros((1, 1, 3, 1, L))
    for k in range(L):
        z[0, 0, :, 0, k] = [-ln3, 0.0, ln3]
    w = oracle.normalize(T2B, z)[0, 0, :, 0, :]
    # interior (k = 1): (1/4, 1/2, 3/4) / (3/2) = (1/6, 1/3, 1/2)
    np.testing.assert_allclose(w[:, 1], [1 / 6, 1 / 3, 1 / 2], rtol=0, atol=1e-15)
    # left border (k = 0): (-, 1/2, 3/4) / (5/4) = (0, 2/5, 3/5)
    np.testing.assert_allclose(w[:, 0], [0.0, 2 / 5, 3 / 5], rtol=0, atol=1e-15)
    # right border (k = 2): (1/4, 1/2, -) / (3/4) = (1/3, 2/3, 0)
    np.testing.assert_allclose(w[:, 2], [1 / 3, 2 / 3, 0.0], rtol=0, atol=1e-15)


def test_normalize_line_of_length_one_is_identity():
    w = oracle.normalize(T2B, _rand_logits(1, 2, 5, 1))
    assert np.all(w[:, :, 1] == 1.0) and np.all(w[:, :, 0] == 0.0) and np.all(w[:, :, 2] == 0.0)


def test_normalize_monotone_in_own_logit():
    z = np.zeros((1, 1, 3, 1, 3))
    base = oracle.normalize(T2B, z)[0, 0, :, 0, 1]
    z[0, 0, 2, 0, 1] = 1.0
    up = oracle.normalize(T2B, z)[0, 0, :, 0, 1]
    assert up[2] > base[2] and up[0] < base[0] and up[1] < base[1]


def test_normalize_horizontal_uses_frame_line_length():
    # Horizontal directions run lines of length H; the border test is along H.
    h, w = 4, 6
    S, L = _frame(L2R, h, w)
    assert (S, L) == (6, 4)
    ww = oracle.normalize(L2R, _rand_logits(1, 1, S, L))
    assert np.all(ww[0, 0, 0, :, 0] == 0.0) and np.all(ww[0, 0, 2, :, L - 1] == 0.0)


# ----------------------------------------------------------------------------
# Independent dense construction of the unrolled scan, H = G X
# ----------------------------------------------------------------------------

def _to_frame(a, direction):
    """[.., H, W] array frame -> [.., S, L] scan frame."""
    return np.swapaxes(a, -1, -2) if direction in (L2R, R2L) else a


def _dense_scan_plane(direction, x_plane, w_frame, lam_frame, chunk=0):
    """Unrolled form of one plane: G is block lower triangular in scan order
    with G_tt = diag(lam_t) and G_ts = M_t M_{t-1} ... M_{s+1} diag(lam_s),
    M_t the tridiagonal L x L matrix of line t.  Built from explicit dense
    matrix products, independent of the oracle's recurrence loop."""
    S, L = w_frame.shape[1:]
    X = _to_frame(x_plane, direction)                     # [S][L]
    order = list(range(S))[::-1] if direction in (B2T, R2L) else list(range(S))
    K = S if chunk in (0,) or chunk >= S else chunk
    M = []
    for i in order:
        m = np.zeros((L, L))
        for k in range(L):
            for o in range(3):
                nb = k + o - 1
                if 0 <= nb < L:
                    m[k, nb] = w_frame[o, i, k]
        M.append(m)
    G = np.zeros((S * L, S * L))
    for t in range(S):
        for s in range(t + 1):
            if t // K != s // K:
                continue
            P = np.eye(L)
            for r in range(s + 1, t + 1):
                P = M[r] @ P
            G[t * L:(t + 1) * L, s * L:(s + 1) * L] = P @ np.diag(lam_frame[order[s]])
    xs = np.concatenate([X[i] for i in order])
    hs = G @ xs
    H = np.zeros((S, L))
    for t, i in enumerate(order):
        H[i] = hs[t * L:(t + 1) * L]
    return np.swapaxes(H, 0, 1) if direction in (L2R, R2L) else H


def _random_stochastic_w(S, L):
    """Random positive tridiagonal rows normalised over the valid neighbours."""
    w = rng.uniform(0.05, 1.0, size=(3, S, L))
    w[0, :, 0] = 0.0
    w[2, :, L - 1] = 0.0
    return w / w.sum(axis=0, keepdims=True)


@pytest.mark.parametrize("direction", [T2B, B2T, L2R, R2L])
@pytest.mark.parametrize("hw", [(16, 16), (7, 5), (5, 7), (1, 6), (6, 1)])
def test_scan_matches_dense_unrolled_form(direction, hw):
    h, w = hw
    S, L = _frame(direction, h, w)
    x = rng.normal(size=(1, 1, h, w))
    wf = _random_stochastic_w(S, L)
    lam = rng.uniform(0, 1, size=(1, 1, S, L))
    got = oracle.scan(direction, x, wf[None, None], lam, wts_are_logits=False)
    ref = _dense_scan_plane(direction, x[0, 0], wf, lam[0, 0])
    np.testing.assert_allclose(got[0, 0], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("direction", [T2B, B2T, L2R, R2L])
@pytest.mark.parametrize("chunk", [1, 3, 8])
def test_chunked_scan_matches_dense_unrolled_form(direction, chunk):
    h, w = 10, 6
    S, L = _frame(direction, h, w)
    x = rng.normal(size=(1, 1, h, w))
    wf = _random_stochastic_w(S, L)
    lam = rng.uniform(0, 1, size=(1, 1, S, L))
    got = oracle.scan(direction, x, wf[None, None], lam, chunk=chunk, wts_are_logits=False)
    ref = _dense_scan_plane(direction, x[0, 0], wf, lam[0, 0], chunk=chunk)
    np.testing.assert_allclose(got[0, 0], ref, rtol=0, atol=1e-12)


def test_logit_path_equals_prenormalised_path():
    h, w = 9, 11
    for d in range(4):
        S, L = _frame(d, h, w)
        x = rng.normal(size=(2, 3, h, w))
        z = _rand_logits(2, 3, S, L)
        lam = rng.uniform(size=(2, 3, S, L))
        a = oracle.scan(d, x, z, lam)
        b = oracle.scan(d, x, oracle.normalize(d, z), lam, wts_are_logits=False)
        np.testing.assert_array_equal(a, b)


# ----------------------------------------------------------------------------
# Exact rational arithmetic on a tiny case
# ----------------------------------------------------------------------------

def test_exact_rational_three_by_three():
    """Logits in {-ln 3, 0, ln 3} give rational weights (sigmoids 1/4, 1/2, 3/4);
    rational lam and x then give an exactly known h, built here by the dense
    unrolled form in Fractions (T2B and L2R)."""
    ln3 = math.log(3.0)
    sig = {-1: Fraction(1, 4), 0: Fraction(1, 2), 1: Fraction(3, 4)}
    h = w = 3
    code = rng.integers(-1, 2, size=(3, h, w))              # logit codes per (o, i, k)
    z = np.where(code == 1, ln3, np.where(code == -1, -ln3, 0.0))
    lam_num = rng.integers(1, 5, size=(h, w))
    x_int = rng.integers(-3, 4, size=(h, w))
    for d in (T2B, L2R):
        S, L = _frame(d, h, w)
        X = x_int.T if d == L2R else x_int
        # exact weights
        W = [[[Fraction(0)] * 3 for _ in range(L)] for _ in range(S)]
        for i in range(S):
            for k in range(L):
                valid = [0 <= k + o - 1 < L for o in range(3)]
                tot = sum(sig[int(code[o, i, k])] for o in range(3) if valid[o])
                for o in range(3):
                    W[i][k][o] = sig[int(code[o, i, k])] / tot if valid[o] else Fraction(0)
        hprev = None
        exact = [[Fraction(0)] * L for _ in range(S)]
        for i in range(S):
            cur = []
            for k in range(L):
                acc = Fraction(int(lam_num[i, k]), 4) * int(X[i, k])
                if hprev is not None:
                    for o in range(3):
                        nb = k + o - 1
                        if 0 <= nb < L:
                            acc += W[i][k][o] * hprev[nb]
                cur.append(acc)
            exact[i] = cur
            hprev = cur
        got = oracle.scan(d, x_int[None, None].astype(float), z[None, None],
                          (lam_num / 4.0)[None, None])[0, 0]
        got_f = got.T if d == L2R else got
        for i in range(S):
            for k in range(L):
                assert abs(got_f[i, k] - float(exact[i][k])) <= 1e-14 * max(1.0, abs(float(exact[i][k])))


# ----------------------------------------------------------------------------
# Closed forms
# ----------------------------------------------------------------------------

def _scan_step_index(direction, h, w):
    """Scan step t of every array position (i, j)."""
    ii, jj = np.meshgrid(np.arange(h), np.arange(w), indexing="ij")
    return {T2B: ii, B2T: h - 1 - ii, L2R: jj, R2L: w - 1 - jj}[direction]


@pytest.mark.parametrize("direction", [T2B, B2T, L2R, R2L])
@pytest.mark.parametrize("chunk", [0, 1, 4, 5, 100])
def test_constant_input_closed_form(direction, chunk):
    # lam = 1 and x = c: h at scan step t is ((t mod K) + 1) c for any logits,
    # because every row of w sums to 1.
    h, w, c = 12, 9, 0.75
    S, L = _frame(direction, h, w)
    x = np.full((2, 2, h, w), c)
    z = _rand_logits(2, 2, S, L, scale=3.0)
    lam = np.ones((2, 2, S, L))
    got = oracle.scan(direction, x, z, lam, chunk=chunk)
    K = S if chunk == 0 or chunk >= S else chunk
    t = _scan_step_index(direction, h, w)
    np.testing.assert_allclose(got, np.broadcast_to(((t % K) + 1) * c, got.shape), rtol=1e-14)


def test_forward4_constant_input_closed_form():
    # Merged: (i+1) + (H-i) + (j+1) + (W-j) = H + W + 2 times c.
    h, w, c = 8, 13, -1.5
    x = np.full((1, 3, h, w), c)
    zs = [_rand_logits(1, 3, *_frame(d, h, w)) for d in range(4)]
    ls = [np.ones((1, 3) + _frame(d, h, w)) for d in range(4)]
    y = oracle.forward4(x, zs, ls)
    np.testing.assert_allclose(y, (h + w + 2) * c, rtol=1e-14)
    # chunk_len 4 divides both sides: each direction contributes (t mod 4) + 1,
    # which sums to 2 (K + 1) per axis pair when K divides H and W.
    h2, w2 = 8, 12
    x2 = np.full((1, 1, h2, w2), c)
    zs2 = [_rand_logits(1, 1, *_frame(d, h2, w2)) for d in range(4)]
    ls2 = [np.ones((1, 1) + _frame(d, h2, w2)) for d in range(4)]
    y2 = oracle.forward4(x2, zs2, ls2, chunk=4)
    np.testing.assert_allclose(y2, 2 * (4 + 1) * c, rtol=1e-14)


def test_line_indicator_gives_all_ones_downstream():
    # x = 1 on one line s (lam = 1) and 0 elsewhere: every later line in scan
    # order is the product of row-stochastic matrices applied to a vector of
    # ones, hence exactly 1 everywhere; earlier lines are 0.
    h, w = 10, 7
    for d in range(4):
        S, L = _frame(d, h, w)
        s = 3
        xf = np.zeros((S, L))
        xf[s] = 1.0
        x = _to_frame(xf, d)[None, None]
        z = _rand_logits(1, 1, S, L, scale=2.0)
        got = _to_frame(oracle.scan(d, np.ascontiguousarray(x), z, np.ones((1, 1, S, L)))[0, 0], d)
        after = range(s, S) if d in (T2B, L2R) else range(0, s + 1)
        before = range(0, s) if d in (T2B, L2R) else range(s + 1, S)
        for i in after:
            np.testing.assert_allclose(got[i], 1.0, rtol=0, atol=1e-14)
        for i in before:
            assert np.all(got[i] == 0.0)


@pytest.mark.parametrize("direction", [T2B, B2T, L2R, R2L])
@pytest.mark.parametrize("chunk", [0, 3])
def test_line_length_one_reduces_to_cumsum(direction, chunk):
    # L = 1 forces w = [1]: the scan is a running sum of lam * x along the scan.
    if direction in (T2B, B2T):
        h, w = 11, 1
    else:
        h, w = 1, 11
    S, L = _frame(direction, h, w)
    x = rng.normal(size=(1, 2, h, w))
    lam = rng.uniform(size=(1, 2, S, L))
    got = _to_frame(oracle.scan(direction, x, _rand_logits(1, 2, S, L), lam, chunk=chunk), direction)
    u = lam * _to_frame(x, direction)                     # [1,2,S,1]
    if direction in (B2T, R2L):
        u = u[:, :, ::-1]
    K = S if chunk == 0 else chunk
    ref = np.concatenate([np.cumsum(u[:, :, a:a + K], axis=2) for a in range(0, S, K)], axis=2)
    if direction in (B2T, R2L):
        ref = ref[:, :, ::-1]
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_chunk_of_one_is_lam_times_x():
    h, w = 6, 5
    for d in range(4):
        S, L = _frame(d, h, w)
        x = rng.normal(size=(1, 1, h, w))
        lam = rng.uniform(size=(1, 1, S, L))
        got = oracle.scan(d, x, _rand_logits(1, 1, S, L), lam, chunk=1)
        np.testing.assert_array_equal(got, x * _to_frame(lam, d))


# ----------------------------------------------------------------------------
# Structure of the unrolled operator
# ----------------------------------------------------------------------------

def test_cone_support_of_impulse_response():
    # G_ts[k, m] > 0 exactly when |k - m| <= t - s: a unit impulse at line s,
    # position m reaches position k of line t iff it is inside the cone.
    h, w = 9, 11
    d = T2B
    S, L = _frame(d, h, w)
    z = _rand_logits(1, 1, S, L)
    s, m = 2, 5
    x = np.zeros((1, 1, h, w))
    x[0, 0, s, m] = 1.0
    got = oracle.scan(d, x, z, np.ones((1, 1, S, L)))[0, 0]
    for t in range(S):
        for k in range(L):
            inside = t >= s and abs(k - m) <= t - s
            assert (got[t, k] > 0.0) == inside, (t, k)


def test_stability_bound_and_linearity():
    h, w = 14, 10
    for d in range(4):
        S, L = _frame(d, h, w)
        z = _rand_logits(1, 1, S, L, scale=2.0)
        lam = rng.uniform(size=(1, 1, S, L))
        x1 = rng.normal(size=(1, 1, h, w))
        x2 = rng.normal(size=(1, 1, h, w))
        a, b = 0.7, -2.3
        lhs = oracle.scan(d, a * x1 + b * x2, z, lam)
        rhs = a * oracle.scan(d, x1, z, lam) + b * oracle.scan(d, x2, z, lam)
        np.testing.assert_allclose(lhs, rhs, rtol=0, atol=1e-12)
        # |h_t|_inf <= sum_{s <= t} |lam_s x_s|_inf  (row-stochastic w)
        hf = _to_frame(oracle.scan(d, x1, z, lam)[0, 0], d)
        uf = np.abs(lam[0, 0] * _to_frame(x1[0, 0], d)).max(axis=1)
        order = list(range(S))[::-1] if d in (B2T, R2L) else list(range(S))
        bound = np.cumsum([uf[i] for i in order])
        for t, i in enumerate(order):
            assert np.abs(hf[i]).max() <= bound[t] + 1e-12


# ----------------------------------------------------------------------------
# Symmetries: reversal and transposition
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("chunk", [0, 4])
def test_reversed_scan_is_forward_scan_of_flipped_input(chunk):
    h, w = 12, 7
    x = rng.normal(size=(2, 2, h, w))
    for fwd, rev, axis in ((T2B, B2T, 2), (L2R, R2L, 3)):
        S, L = _frame(fwd, h, w)
        z = _rand_logits(2, 2, S, L)
        lam = rng.uniform(size=(2, 2, S, L))
        if chunk and S % chunk:
            continue
        got = oracle.scan(rev, x, z, lam, chunk=chunk)
        ref = np.flip(oracle.scan(fwd, np.flip(x, axis).copy(), np.flip(z, 3).copy(),
                                  np.flip(lam, 2).copy(), chunk=chunk), axis)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


def test_horizontal_scan_is_vertical_scan_of_transposed_input():
    h, w = 6, 10
    x = rng.normal(size=(1, 3, h, w))
    for hd, vd in ((L2R, T2B), (R2L, B2T)):
        S, L = _frame(hd, h, w)
        z = _rand_logits(1, 3, S, L)
        lam = rng.uniform(size=(1, 3, S, L))
        got = oracle.scan(hd, x, z, lam)
        xt = np.ascontiguousarray(np.swapaxes(x, 2, 3))
        ref = np.swapaxes(oracle.scan(vd, xt, z, lam), 2, 3)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-13)


# ----------------------------------------------------------------------------
# Channel-shared w, merge, projections
# ----------------------------------------------------------------------------

def test_shared_w_equals_broadcast_per_channel_w():
    h, w, c = 7, 9, 4
    for d in range(4):
        S, L = _frame(d, h, w)
        x = rng.normal(size=(2, c, h, w))
        z1 = _rand_logits(2, 1, S, L)
        lam = rng.uniform(size=(2, c, S, L))
        a = oracle.scan(d, x, z1, lam)
        b = oracle.scan(d, x, np.repeat(z1, c, axis=1), lam)
        np.testing.assert_array_equal(a, b)


def test_forward4_is_sum_of_directions():
    h, w = 9, 6
    x = rng.normal(size=(2, 2, h, w))
    zs = [_rand_logits(2, 2, *_frame(d, h, w)) for d in range(4)]
    ls = [rng.uniform(size=(2, 2) + _frame(d, h, w)) for d in range(4)]
    y = oracle.forward4(x, zs, ls, chunk=3)
    ref = sum(oracle.scan(d, x, zs[d], ls[d], chunk=3) for d in range(4))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-13)


def test_project_matches_einsum():
    x = rng.normal(size=(2, 37, 5, 6))
    wt = rng.normal(size=(8, 37))
    np.testing.assert_allclose(oracle.project(x, wt), np.einsum("pc,nchw->nphw", wt, x),
                               rtol=1e-13, atol=1e-13)


def test_proxy_forward4_composition():
    n, c, cp, h, w = 1, 20, 4, 6, 7
    x = rng.normal(size=(n, c, h, w))
    wd = rng.normal(size=(cp, c))
    wu = rng.normal(size=(c, cp))
    zs = [_rand_logits(n, 1, *_frame(d, h, w)) for d in range(4)]
    ls = [rng.uniform(size=(n, cp) + _frame(d, h, w)) for d in range(4)]
    y = oracle.proxy_forward4(x, wd, wu, zs, ls)
    xp = np.einsum("pc,nchw->nphw", wd, x)
    ref = np.einsum("cp,nphw->nchw", wu, oracle.forward4(xp, zs, ls))
    np.testing.assert_allclose(y, ref, rtol=0, atol=1e-12)


def test_empty_inputs():
    for d in range(4):
        x = np.zeros((0, 2, 4, 4))
        S, L = _frame(d, 4, 4)
        out = oracle.scan(d, x, np.zeros((0, 2, 3, S, L)), np.zeros((0, 2, S, L)))
        assert out.shape == (0, 2, 4, 4)


def test_bad_arguments_are_rejected():
    x = np.zeros((1, 2, 4, 4))
    with pytest.raises(ValueError):
        oracle.scan(T2B, x, np.zeros((1, 3, 3, 4, 4)), np.zeros((1, 2, 4, 4)))
    with pytest.raises(ValueError):
        oracle.scan(T2B, x, np.zeros((1, 2, 3, 4, 4)), np.zeros((1, 2, 4, 4)), chunk=-1)
