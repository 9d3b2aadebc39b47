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
