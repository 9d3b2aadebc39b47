"""Pins for the per-direction variant of the oracle (per-direction lambda /
u, "Key design 2"'s learnable merger as per-direction gates).

The variant oracle is a sum of single-direction oracle calls; it is checked
against the dense closed form with per-direction tensors (tests/bruteforce.py,
an independent formulation), and against the shared-tensor oracle when every
direction gets the same slab.
"""
import numpy as np
import pytest

import oracle
from bruteforce import bruteforce_fwd


def case(rng, B, C, H, W, dirs, cpw, lam_dir, u_dir):
    nd = bin(dirs).count("1")
    x = rng.standard_normal((B, C, H, W))
    lam = rng.random((nd, B, C, H, W) if lam_dir else (B, C, H, W))
    u = rng.random((nd, B, C, H, W) if u_dir else (B, C, H, W))
    w = rng.standard_normal((nd, B, C // cpw, 3, H, W))
    return x, w, lam, u


@pytest.mark.parametrize("lam_dir,u_dir", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("H,W,dirs,g,cpw", [(5, 6, 15, 1, 1), (6, 4, 15, 2, 2), (4, 4, 5, 1, 1),
                                            (3, 7, 10, 1, 1), (8, 8, 12, 4, 2)])
def test_variant_matches_dense_closed_form(H, W, dirs, g, cpw, lam_dir, u_dir):
    rng = np.random.default_rng(H * 13 + W + dirs + g)
    x, w, lam, u = case(rng, 2, 2 * cpw, H, W, dirs, cpw, lam_dir, u_dir)
    y0 = oracle.scan_fwd_dirs(x, w, lam, u, dirs=dirs, groups=g, cpw=cpw)
    y1 = bruteforce_fwd(x, w, lam, u, dirs=dirs, groups=g, cpw=cpw, check=False)
    np.testing.assert_allclose(y0, y1, rtol=0, atol=1e-12 * max(1.0, np.abs(y1).max()))


def test_replicated_slabs_equal_shared_call():
    rng = np.random.default_rng(1)
    x, w, lam, u = case(rng, 2, 4, 7, 9, 15, 2, False, False)
    y_shared = oracle.scan_fwd(x, w, lam, u, cpw=2)
    rep = lambda a: np.stack([a] * 4)
    y_dir = oracle.scan_fwd_dirs(x, w, rep(lam), rep(u), cpw=2)
    np.testing.assert_allclose(y_dir, y_shared, rtol=0, atol=1e-12 * np.abs(y_shared).max())


def test_gate_selects_one_direction():
    """u_d = 1 for one direction and 0 for the others gives that direction alone."""
    rng = np.random.default_rng(2)
    x, w, lam, _ = case(rng, 1, 2, 6, 6, 15, 1, True, False)
    for d in range(4):
        u = np.zeros((4, 1, 2, 6, 6))
        u[d] = 1.0
        y = oracle.scan_fwd_dirs(x, w, lam, u)
        y_one = oracle.scan_fwd(x, w[d:d + 1], lam[d], np.ones_like(x), dirs=1 << d)
        np.testing.assert_allclose(y, y_one, rtol=0, atol=1e-13 * np.abs(y_one).max())


# ------------------------------------------------------------ backward of the variant
# Evidence independent of the oracle's backward: y is linear in x, in each
# lam_d and in each u_d, so <g, v> must equal <gy, y(input := v)> with the
# dense closed form (tests/bruteforce.py) evaluated at v; the tap gradient is
# checked against central differences of the dense form along random
# directions.

def bf_loss(x, w, lam, u, gy, **kw):
    return float((bruteforce_fwd(x, w, lam, u, check=False, **kw) * gy).sum())


@pytest.mark.parametrize("lam_dir,u_dir", [(True, False), (False, True), (True, True)])
@pytest.mark.parametrize("H,W,dirs,g,cpw", [(5, 6, 15, 1, 1), (6, 4, 15, 2, 2), (4, 4, 5, 1, 1),
                                            (3, 7, 10, 1, 1), (8, 8, 12, 4, 2)])
def test_variant_bwd_linear_inputs_exact(H, W, dirs, g, cpw, lam_dir, u_dir):
    rng = np.random.default_rng(H * 17 + W + dirs * 3 + g)
    x, w, lam, u = case(rng, 2, 2 * cpw, H, W, dirs, cpw, lam_dir, u_dir)
    gy = rng.standard_normal(x.shape)
    kw = dict(dirs=dirs, groups=g, cpw=cpw)
    gx, _, glam, gu = oracle.scan_bwd_dirs(x, w, lam, u, gy, **kw)
    assert glam.shape == lam.shape and gu.shape == u.shape
    for _ in range(2):
        vx = rng.standard_normal(x.shape)
        vl = rng.standard_normal(lam.shape)
        vu = rng.standard_normal(u.shape)
        for got, v, args in ((gx, vx, (vx, w, lam, u)), (glam, vl, (x, w, vl, u)), (gu, vu, (x, w, lam, vu))):
            want = bf_loss(*args, gy, **kw)
            assert abs(float((got * v).sum()) - want) <= 1e-11 * max(1.0, abs(want))


@pytest.mark.parametrize("lam_dir,u_dir", [(True, True), (True, False)])
@pytest.mark.parametrize("H,W,dirs,g,cpw", [(6, 5, 15, 1, 1), (6, 6, 9, 3, 2), (5, 7, 6, 1, 1)])
def test_variant_bwd_tap_gradient_directional_derivative(H, W, dirs, g, cpw, lam_dir, u_dir):
    rng = np.random.default_rng(H * 29 + W + dirs)
    x, w, lam, u = case(rng, 1, 2 * cpw, H, W, dirs, cpw, lam_dir, u_dir)
    w = 2.0 * w
    gy = rng.standard_normal(x.shape)
    kw = dict(dirs=dirs, groups=g, cpw=cpw)
    gw = oracle.scan_bwd_dirs(x, w, lam, u, gy, **kw)[1]
    for _ in range(3):
        v = rng.standard_normal(w.shape)
        eps = 1e-5
        fd = (bf_loss(x, w + eps * v, lam, u, gy, **kw) - bf_loss(x, w - eps * v, lam, u, gy, **kw)) / (2 * eps)
        assert abs(float((gw * v).sum()) - fd) <= 1e-7 * max(1.0, abs(fd))


def test_variant_bwd_replicated_slabs_equal_shared_call():
    """Every direction given the same lam and u: the per-slab gradients sum
    to the shared-tensor gradients, and gx, gw are unchanged."""
    rng = np.random.default_rng(4)
    x, w, lam, u = case(rng, 2, 4, 7, 9, 15, 2, False, False)
    gy = rng.standard_normal(x.shape)
    shared = oracle.scan_bwd(x, w, lam, u, gy, cpw=2)
    rep = lambda a: np.stack([a] * 4)
    gx, gw, glam, gu = oracle.scan_bwd_dirs(x, w, rep(lam), rep(u), gy, cpw=2)
    for got, want in ((gx, shared[0]), (gw, shared[1]), (glam.sum(0), shared[2]), (gu.sum(0), shared[3])):
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12 * max(1.0, np.abs(want).max()))


def _linear_pins_hold(gx, glam, gu, x, w, lam, u, gy, kw, rng):
    vx, vl, vu = (rng.standard_normal(a.shape) for a in (x, lam, u))
    for got, v, args in ((gx, vx, (vx, w, lam, u)), (glam, vl, (x, w, vl, u)), (gu, vu, (x, w, lam, vu))):
        want = bf_loss(*args, gy, **kw)
        if abs(float((got * v).sum()) - want) > 1e-11 * max(1.0, abs(want)):
            return False
    return True


# plausible mistakes in assembling the per-direction gradients
VARIANT_BWD_MUTANTS = {
    "gx_drops_last_direction": lambda gx, glam, gu, parts: (gx - parts[-1][0], glam, gu),
    "glam_slabs_reversed": lambda gx, glam, gu, parts: (gx, glam[::-1].copy(), gu),
    "gu_slabs_reversed": lambda gx, glam, gu, parts: (gx, glam, gu[::-1].copy()),
    "gu_every_slab_gets_the_sum": lambda gx, glam, gu, parts: (gx, glam, np.stack([gu.sum(0)] * len(gu))),
    "gx_counts_first_direction_twice": lambda gx, glam, gu, parts: (gx + parts[0][0], glam, gu),
    "glam_summed_into_every_slab": lambda gx, glam, gu, parts: (gx, np.stack([glam.sum(0)] * len(glam)), gu),
}


@pytest.mark.parametrize("name", sorted(VARIANT_BWD_MUTANTS))
def test_variant_bwd_pins_catch_planted_mistakes(name):
    rng = np.random.default_rng(9)
    H, W, dirs, g, cpw = 5, 6, 15, 1, 1
    x, w, lam, u = case(rng, 2, 2, H, W, dirs, cpw, True, True)
    gy = rng.standard_normal(x.shape)
    kw = dict(dirs=dirs, groups=g, cpw=cpw)
    gx, _, glam, gu = oracle.scan_bwd_dirs(x, w, lam, u, gy, **kw)
    assert _linear_pins_hold(gx, glam, gu, x, w, lam, u, gy, kw, np.random.default_rng(1))
    parts = [oracle.scan_bwd(x, w[s:s + 1], lam[s], u[s], gy, dirs=1 << d, groups=g, cpw=cpw)
             for s, d in enumerate(range(4))]
    bad = VARIANT_BWD_MUTANTS[name](gx, glam, gu, parts)
    assert not _linear_pins_hold(*bad, x, w, lam, u, gy, kw, np.random.default_rng(1))
