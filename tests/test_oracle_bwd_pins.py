"""Pins for the fp64 oracle's backward pass (the exact vector-Jacobian product).

The evidence does not come from the oracle itself:

* central finite differences of the dense closed form in ``bruteforce.py``
  (an independent forward) for the raw-tap gradient, element by element on
  tiny grids and along random directions on larger ones;
* exact directional derivatives for x, lambda and u: y is linear in each of
  them separately, so <g, v> must equal <gy, y(v)> with the dense closed form
  evaluated at v in place of that input;
* Theorem 1 ("Key design 1"): with x = lambda = u = 1 the output is the same
  constant for every choice of taps, so the raw-tap gradient vanishes;
* taps the forward never reads (missing border neighbours, first lines of
  local groups, lines of length 1) get exactly zero gradient.
"""
import numpy as np
import pytest

import oracle
from bruteforce import bruteforce_fwd


def rand_case(rng, B, C, H, W, dirs, cpw, wscale=1.0):
    nd = bin(dirs).count("1")
    x = rng.standard_normal((B, C, H, W))
    lam = rng.random((B, C, H, W))
    u = rng.random((B, C, H, W))
    w = wscale * rng.standard_normal((nd, B, C // cpw, 3, H, W))
    gy = rng.standard_normal((B, C, H, W))
    return x, w, lam, u, gy


def bf_loss(x, w, lam, u, gy, **kw):
    return float((bruteforce_fwd(x, w, lam, u, check=False, **kw) * gy).sum())


def fd_tap_grad(x, w, lam, u, gy, eps=1e-6, **kw):
    g = np.zeros_like(w)
    for idx in np.ndindex(w.shape):
        wp = w.copy()
        wp[idx] += eps
        wm = w.copy()
        wm[idx] -= eps
        g[idx] = (bf_loss(x, wp, lam, u, gy, **kw) - bf_loss(x, wm, lam, u, gy, **kw)) / (2 * eps)
    return g


@pytest.mark.parametrize("H,W,dirs,g,cpw", [
    (4, 5, 15, 1, 1), (5, 4, 15, 1, 2), (3, 3, 1, 1, 1), (3, 4, 2, 1, 1), (4, 3, 4, 1, 1),
    (3, 4, 8, 1, 1), (4, 4, 15, 2, 1), (6, 6, 5, 3, 2), (4, 6, 10, 2, 1), (1, 4, 15, 1, 1),
    (4, 1, 15, 1, 1), (2, 2, 15, 2, 1)])
def test_tap_gradient_matches_finite_differences_of_dense_form(H, W, dirs, g, cpw):
    rng = np.random.default_rng(H * 100 + W * 10 + dirs + g)
    x, w, lam, u, gy = rand_case(rng, 1, 2 * cpw, H, W, dirs, cpw)
    kw = dict(dirs=dirs, groups=g, cpw=cpw)
    gw = oracle.scan_bwd(x, w, lam, u, gy, **kw)[1]
    fd = fd_tap_grad(x, w, lam, u, gy, **kw)
    np.testing.assert_allclose(gw, fd, rtol=0, atol=1e-7 * max(1.0, np.abs(fd).max()))


@pytest.mark.parametrize("H,W,dirs,g,cpw", [(8, 8, 15, 1, 1), (8, 6, 15, 2, 2), (6, 9, 9, 3, 1),
                                            (7, 5, 6, 1, 4)])
def test_tap_gradient_directional_derivative(H, W, dirs, g, cpw):
    rng = np.random.default_rng(H * 31 + W + dirs)
    x, w, lam, u, gy = rand_case(rng, 2, 4, H, W, dirs, cpw, wscale=2.0)
    kw = dict(dirs=dirs, groups=g, cpw=cpw)
    gw = oracle.scan_bwd(x, w, lam, u, gy, **kw)[1]
    for _ in range(3):
        v = rng.standard_normal(w.shape)
        eps = 1e-5
        fd = (bf_loss(x, w + eps * v, lam, u, gy, **kw) - bf_loss(x, w - eps * v, lam, u, gy, **kw)) / (2 * eps)
        assert abs(float((gw * v).sum()) - fd) <= 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("H,W,dirs,g,cpw", [(5, 7, 15, 1, 1), (8, 8, 15, 4, 2), (6, 4, 3, 2, 1),
                                            (4, 6, 12, 3, 1), (1, 6, 15, 1, 1), (7, 1, 3, 7, 1)])
def test_linear_input_gradients_are_exact(H, W, dirs, g, cpw):
    """y is linear in x, in lambda and in u: <g_in, v> == <gy, y(in := v)>."""
    rng = np.random.default_rng(H * 7 + W * 3 + dirs + g)
    x, w, lam, u, gy = rand_case(rng, 2, 4, H, W, dirs, cpw)
    kw = dict(dirs=dirs, groups=g, cpw=cpw)
    gx, _, glam, gu = oracle.scan_bwd(x, w, lam, u, gy, **kw)
    for _ in range(2):
        v = rng.standard_normal(x.shape)
        for got, args in ((gx, (v, w, lam, u)), (glam, (x, w, v, u)), (gu, (x, w, lam, v))):
            want = bf_loss(*args, gy, **kw)
            assert abs(float((got * v).sum()) - want) <= 1e-11 * max(1.0, np.abs(want))


@pytest.mark.parametrize("H,W,g", [(6, 5, 1), (8, 8, 2), (4, 12, 4), (1, 7, 1)])
def test_ones_input_gives_zero_tap_gradient(H, W, g):
    """x = lambda = u = 1: y == (H/g + 1) + (W/g + 1) for any taps (Theorem 1)."""
    rng = np.random.default_rng(H + W + g)
    one = np.ones((2, 3, H, W))
    w = 3 * rng.standard_normal((4, 2, 3, 3, H, W))
    gy = rng.standard_normal(one.shape)
    gx, gw, glam, gu = oracle.scan_bwd(one, w, one, one, gy, groups=g)
    assert np.abs(gw).max() <= 1e-12 * np.abs(gy).max() * H * W
    np.testing.assert_allclose(gu, gy * ((H // g + 1) + (W // g + 1)), rtol=1e-13, atol=0)
    np.testing.assert_allclose(gx, glam, rtol=1e-13, atol=1e-13)


def test_unread_taps_have_zero_gradient():
    rng = np.random.default_rng(3)
    H, W, g = 6, 8, 2
    x, w, lam, u, gy = rand_case(rng, 1, 2, H, W, 15, 1)
    gw = oracle.scan_bwd(x, w, lam, u, gy, groups=g)[1][:, 0, 0]   # [4][3][H][W]
    # first line of every group
    for r in range(0, H, H // g):
        assert not gw[0, :, r].any()             # TB: rows 0, 3
    for r in range(H - 1, -1, -(H // g)):
        assert not gw[1, :, r].any()             # BT: rows 5, 2
    for q in range(0, W, W // g):
        assert not gw[2, :, :, q].any()          # LR
    for q in range(W - 1, -1, -(W // g)):
        assert not gw[3, :, :, q].any()          # RL
    # missing border neighbours: tap 0 at position 0, tap 2 at the last position
    assert not gw[0:2, 0, :, 0].any() and not gw[0:2, 2, :, W - 1].any()
    assert not gw[2:4, 0, 0, :].any() and not gw[2:4, 2, H - 1, :].any()
    # every tap that is read has a non-zero gradient for generic data
    read = np.ones_like(gw, dtype=bool)
    read[np.where(gw == 0)] = False
    assert read.sum() > 0.5 * gw.size


def test_length_one_lines_have_zero_tap_gradient():
    """A line of one position has the single weight 1, whatever its tap."""
    rng = np.random.default_rng(4)
    x, w, lam, u, gy = rand_case(rng, 1, 1, 1, 6, 15, 1)
    gw = oracle.scan_bwd(x, w, lam, u, gy)[1]
    assert not gw[0:2].any()          # TB and BT: the only line starts its group
    assert not gw[2:4].any()          # LR and RL lines have length H = 1


def test_bwd_bad_arguments_rejected():
    rng = np.random.default_rng(5)
    x, w, lam, u, gy = rand_case(rng, 1, 2, 4, 4, 15, 1)
    with pytest.raises(ValueError):
        oracle.scan_bwd(x, w, lam, u, gy, groups=3)
    with pytest.raises(ValueError):
        oracle.scan_bwd(x, w, lam, u, gy[..., :3])
