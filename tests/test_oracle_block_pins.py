"""Pins of the oracle's compressed block (oracle.block_fwd), no GPU.

The block is read from the GSPN-2 response (*Relate Compressive Proxy
Dimension to Low-rank Approximation*) and the C-GSPN abstract: a per-pixel
linear layer from C channels to x_proxy and to the scan's raw taps, lambda
and u; the scan over x_proxy; a per-pixel linear layer back to C channels.

- A pixel-by-pixel composition with pure-Python loops for both linear
  layers and the dense closed-form scan checker (tests/bruteforce.py) pins
  the row order of the input projection, the tap-slab layout and the output
  projection on tiny grids.
- A bias channel turns the generated taps, lambda and u into constants; the
  block then equals the output projection of the (separately pinned) scan
  oracle on those constants.
- round_bf16 is pinned on hand-picked ties and on torch's own conversion.
"""
import math

import numpy as np
import pytest

import oracle
from bruteforce import bruteforce_fwd


def _block_loops(x, w_in, w_out, dirs, groups, cpw, rnd=None, norm=False):
    """The block by pixel loops; rnd (if given) rounds each generated value
    and each scan output one at a time, the places a block that stores its
    intermediates in a narrower dtype rounds them.  norm: each pixel's scan
    output is divided by its root mean square over the proxy channels
    (sqrt(sum_q y_q^2 / C_proxy + eps)) before the output projection."""
    rnd = rnd or (lambda v: v)
    B, C, H, W = x.shape
    Cp = w_out.shape[1]
    nd = bin(dirs).count("1")
    Cw = Cp // cpw
    rows = w_in.shape[0]
    g = np.zeros((B, rows, H, W))
    for b in range(B):
        for r in range(rows):
            for i in range(H):
                for j in range(W):
                    s = 0.0
                    for c in range(C):
                        s += w_in[r, c] * x[b, c, i, j]
                    g[b, r, i, j] = rnd(s)
    xp = g[:, :Cp]
    taps = np.zeros((nd, B, Cw, 3, H, W))
    for sl in range(nd):
        for k in range(Cw):
            for t in range(3):
                taps[sl, :, k, t] = g[:, Cp + (sl * Cw + k) * 3 + t]
    base = Cp + nd * Cw * 3
    lam = g[:, base:base + Cp]
    u = g[:, base + Cp:base + 2 * Cp]
    y = bruteforce_fwd(xp, taps, lam, u, dirs=dirs, groups=groups, cpw=cpw)
    y = np.vectorize(rnd)(y)
    if norm:
        for b in range(B):
            for i in range(H):
                for j in range(W):
                    ms = sum(y[b, q, i, j] ** 2 for q in range(Cp)) / Cp
                    for q in range(Cp):
                        y[b, q, i, j] /= math.sqrt(ms + oracle.BLOCK_NORM_EPS)
    z = np.zeros((B, C, H, W))
    for b in range(B):
        for c in range(C):
            for i in range(H):
                for j in range(W):
                    z[b, c, i, j] = sum(w_out[c, q] * y[b, q, i, j] for q in range(Cp))
    return z


@pytest.mark.parametrize("case", [
    (1, 3, 2, 3, 4, 15, 1, 1),
    (2, 4, 4, 4, 3, 15, 1, 2),
    (1, 5, 2, 4, 4, 6, 2, 2),     # BT and LR only, groups of two lines
    (1, 2, 3, 2, 5, 9, 1, 3),     # TB and RL, one weight set for three channels
])
@pytest.mark.parametrize("norm", [False, True])
def test_block_matches_pixel_loops_and_dense_scan(case, norm):
    B, C, Cp, H, W, dirs, groups, cpw = case
    rng = np.random.default_rng(sum(case))
    x = rng.standard_normal((B, C, H, W))
    w_in = rng.standard_normal((oracle.block_rows(Cp, dirs, cpw), C)) * 0.7
    w_out = rng.standard_normal((C, Cp))
    z = oracle.block_fwd(x, w_in, w_out, dirs=dirs, groups=groups, cpw=cpw, norm=norm)
    ref = _block_loops(x, w_in, w_out, dirs, groups, cpw, norm=norm)
    np.testing.assert_allclose(z, ref, rtol=1e-11, atol=1e-12)


def test_block_row_blocks_are_distinguished():
    # the pin above would catch a swapped lambda / u block or tap slab: both
    # change the output on generic inputs
    B, C, Cp, H, W, dirs, cpw = 1, 3, 2, 3, 4, 15, 1
    rng = np.random.default_rng(5)
    x = rng.standard_normal((B, C, H, W))
    w_in = rng.standard_normal((oracle.block_rows(Cp, dirs, cpw), C))
    w_out = rng.standard_normal((C, Cp))
    z = oracle.block_fwd(x, w_in, w_out, dirs=dirs, cpw=cpw, norm=False)
    nd, Cw = 4, Cp // cpw
    base = Cp + nd * Cw * 3
    swapped = w_in.copy()
    swapped[base:base + Cp], swapped[base + Cp:] = w_in[base + Cp:], w_in[base:base + Cp]
    assert np.abs(oracle.block_fwd(x, swapped, w_out, dirs=dirs, cpw=cpw, norm=False) - z).max() > 1e-3
    slabs = w_in.copy()
    slabs[Cp:Cp + 6], slabs[Cp + 6:Cp + 12] = w_in[Cp + 6:Cp + 12], w_in[Cp:Cp + 6]
    assert np.abs(oracle.block_fwd(x, slabs, w_out, dirs=dirs, cpw=cpw, norm=False) - z).max() > 1e-3


def test_block_with_constant_generated_tensors_is_the_projected_scan():
    # channel C-1 of x is 1 everywhere: rows that read only it generate
    # constants, and the proxy rows copy channels 0 .. Cp-1
    B, Cp, H, W, dirs, groups, cpw = 2, 4, 6, 5, 15, 1, 2
    C = Cp + 1
    rng = np.random.default_rng(11)
    x = rng.standard_normal((B, C, H, W))
    x[:, C - 1] = 1.0
    nd, Cw = 4, Cp // cpw
    w_in = np.zeros((oracle.block_rows(Cp, dirs, cpw), C))
    w_in[:Cp, :Cp] = np.eye(Cp)
    tap_vals = rng.standard_normal((nd, Cw, 3))
    for sl in range(nd):
        for k in range(Cw):
            for t in range(3):
                w_in[Cp + (sl * Cw + k) * 3 + t, C - 1] = tap_vals[sl, k, t]
    base = Cp + nd * Cw * 3
    lam_vals, u_vals = rng.uniform(0.2, 1.0, Cp), rng.uniform(0.5, 1.5, Cp)
    w_in[base:base + Cp, C - 1] = lam_vals
    w_in[base + Cp:, C - 1] = u_vals
    w_out = rng.standard_normal((C, Cp))
    z = oracle.block_fwd(x, w_in, w_out, dirs=dirs, groups=groups, cpw=cpw, norm=False)
    taps = np.broadcast_to(tap_vals[:, None, :, :, None, None], (nd, B, Cw, 3, H, W))
    lam = np.broadcast_to(lam_vals[None, :, None, None], (B, Cp, H, W))
    u = np.broadcast_to(u_vals[None, :, None, None], (B, Cp, H, W))
    y = oracle.scan_fwd(x[:, :Cp], taps, lam, u, dirs=dirs, groups=groups, cpw=cpw)
    ref = np.einsum("cq,bqhw->bchw", w_out, y)
    np.testing.assert_allclose(z, ref, rtol=1e-12, atol=1e-12)


def test_round_bf16_ties_and_torch():
    one = 1.0
    ulp = 2.0 ** -7
    vals = np.array([one + ulp / 2, one + 3 * ulp / 2, -(one + ulp / 2), 3.0, 0.0, -0.0, 2.0 ** -130])
    want = np.array([one, one + 2 * ulp, -one, 3.0, 0.0, -0.0, 2.0 ** -130])
    np.testing.assert_array_equal(oracle.round_bf16(vals), want)
    torch = pytest.importorskip("torch")
    r = np.random.default_rng(3).standard_normal(4096) * 10.0 ** np.random.default_rng(4).integers(-6, 6, 4096)
    r32 = r.astype(np.float32).astype(np.float64)
    np.testing.assert_array_equal(oracle.round_bf16(r32),
                                  torch.tensor(r32, dtype=torch.float32).to(torch.bfloat16).double().numpy())


def _bf16_scalar(v):
    """One value rounded to bfloat16 by torch's own conversion (through
    float32, round to nearest even), as fp64."""
    torch = pytest.importorskip("torch")
    return float(torch.tensor(float(v), dtype=torch.float32).to(torch.bfloat16).double())


@pytest.mark.parametrize("case", [
    (1, 3, 2, 3, 4, 15, 1, 1),
    (2, 4, 4, 4, 4, 6, 2, 2),
])
def test_block_io_rounding_placement(case):
    # io_round rounds exactly the five stored tensors: x_proxy, the taps,
    # lambda and u as the input projection produces them, and the scan output
    # before the output projection (z itself is left to the caller's dtype)
    B, C, Cp, H, W, dirs, groups, cpw = case
    rng = np.random.default_rng(100 + sum(case))
    x = rng.standard_normal((B, C, H, W))
    w_in = rng.standard_normal((oracle.block_rows(Cp, dirs, cpw), C)) * 0.7
    w_out = rng.standard_normal((C, Cp))
    z = oracle.block_fwd(x, w_in, w_out, dirs=dirs, groups=groups, cpw=cpw, io_round=oracle.round_bf16)
    ref = _block_loops(x, w_in, w_out, dirs, groups, cpw, rnd=_bf16_scalar, norm=True)
    np.testing.assert_allclose(z, ref, rtol=1e-11, atol=1e-12)
    # the rounding is really applied, at both places
    exact = oracle.block_fwd(x, w_in, w_out, dirs=dirs, groups=groups, cpw=cpw)
    assert np.abs(z - exact).max() > 1e-4
    gen_only = _block_loops(x, w_in, w_out, dirs, groups, cpw, rnd=None, norm=True)
    assert np.abs(gen_only - ref).max() > 1e-4


def test_block_norm_removes_the_scale_of_the_proxy():
    # y is linear in x_proxy, so scaling the x_proxy rows of w_in by a > 0
    # scales y by a: with the normalisation z is unchanged (the eps term
    # aside), without it z scales by a
    B, C, Cp, H, W, dirs, cpw = 2, 5, 4, 5, 6, 15, 2
    rng = np.random.default_rng(21)
    x = rng.standard_normal((B, C, H, W))
    w_in = rng.standard_normal((oracle.block_rows(Cp, dirs, cpw), C))
    w_out = rng.standard_normal((C, Cp))
    scaled = w_in.copy()
    scaled[:Cp] *= 7.0
    z = oracle.block_fwd(x, w_in, w_out, dirs=dirs, cpw=cpw)
    np.testing.assert_allclose(oracle.block_fwd(x, scaled, w_out, dirs=dirs, cpw=cpw), z, rtol=1e-6, atol=1e-9)
    zr = oracle.block_fwd(x, w_in, w_out, dirs=dirs, cpw=cpw, norm=False)
    np.testing.assert_allclose(oracle.block_fwd(x, scaled, w_out, dirs=dirs, cpw=cpw, norm=False), 7.0 * zr,
                               rtol=1e-11, atol=1e-12)


def test_block_norm_gives_unit_mean_square_through_identity():
    # with w_out the identity (C = C_proxy) the output of each pixel is the
    # normalised scan output: its mean square over channels is ms / (ms + eps)
    B, Cp, H, W, dirs, cpw = 1, 6, 4, 5, 15, 3
    rng = np.random.default_rng(22)
    x = rng.standard_normal((B, Cp, H, W))
    w_in = rng.standard_normal((oracle.block_rows(Cp, dirs, cpw), Cp))
    z = oracle.block_fwd(x, w_in, np.eye(Cp), dirs=dirs, cpw=cpw)
    y = oracle.block_fwd(x, w_in, np.eye(Cp), dirs=dirs, cpw=cpw, norm=False)
    ms = np.mean(y * y, axis=1)
    np.testing.assert_allclose(np.mean(z * z, axis=1), ms / (ms + oracle.BLOCK_NORM_EPS), rtol=1e-12)
    np.testing.assert_allclose(z * np.sqrt(ms + oracle.BLOCK_NORM_EPS)[:, None], y, rtol=1e-12, atol=1e-14)
