"""The block parity metric catches a misplaced or truncating rounding, no GPU.

A CPU stand-in for a bf16 block is built from the pinned oracle pieces: both
projections as float32 matrix products (fp32 accumulation, like the GPU's
GEMMs), the five stored intermediates (x_proxy, taps, lambda, u and the scan
output y) rounded to bf16, the scan in fp64 on the rounded values, and z
rounded to bf16.  With round-to-nearest-even stores it must pass the metric
that the GPU block test applies (tests/parity.py, block_error and
BLOCK_TOL); with a truncating store of any one stage, or with a stage left
unrounded, it must fail it.
"""
import numpy as np
import pytest

import oracle
from parity import BLOCK_TOL, block_error, block_passes
from linear_spatial_propagation_amd.inputs import BlockInputs


def trunc_bf16(a):
    """bf16 by dropping the low 16 bits of the float32 value (truncation)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    return (f.view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)


def keep_f32(a):
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def stand_in(inp, x, w_in, w_out, r_g, r_y, r_z, norm=True):
    """Block with fp32 GEMMs; r_g rounds the generated tensors, r_y the scan
    output, r_z the block output.  norm: the RMS normalisation of each
    pixel's scan output over the proxy channels, in fp32, applied to the
    projection's fp32 sums.  Returns z and the normalised scan output."""
    B, C, H, W = x.shape
    Cp, nd, Cw = inp.C_proxy, bin(inp.dirs).count("1"), inp.C_proxy // inp.cpw
    g = np.matmul(w_in.astype(np.float32), x.reshape(B, C, H * W).astype(np.float32)).astype(np.float64)
    t0, t1 = Cp, Cp + nd * Cw * 3
    xp = r_g(g[:, :Cp]).reshape(B, Cp, H, W)
    taps = r_g(g[:, t0:t1]).reshape(B, nd, Cw, 3, H, W).transpose(1, 0, 2, 3, 4, 5)
    lam = r_g(g[:, t1:t1 + Cp]).reshape(B, Cp, H, W)
    u = r_g(g[:, t1 + Cp:]).reshape(B, Cp, H, W)
    y = r_y(oracle.scan_fwd(xp, taps, lam, u, dirs=inp.dirs, groups=inp.groups, cpw=inp.cpw))
    y32 = y.reshape(B, Cp, H * W).astype(np.float32)
    inv = np.ones((B, 1, H * W), np.float32)
    if norm:
        inv = np.float32(1.0) / np.sqrt(np.mean(y32 * y32, axis=1, keepdims=True) + np.float32(oracle.BLOCK_NORM_EPS))
    z = (np.matmul(w_out.astype(np.float32), y32) * inv).astype(np.float64)
    y_n = (y32 * inv).astype(np.float64).reshape(B, Cp, H, W)
    return r_z(z).reshape(B, w_out.shape[0], H, W), y_n


SHAPES = [
    # B, C, C_proxy, H, W, groups, cpw
    (2, 96, 32, 16, 16, 1, 4),
    (1, 64, 16, 24, 20, 2, 2),
    (2, 160, 128, 8, 16, 1, 16),
]
R = oracle.round_bf16
MUTANTS = {
    "truncated generated tensors": (trunc_bf16, R, R),
    "truncated scan output": (R, trunc_bf16, R),
    "truncated block output": (R, R, trunc_bf16),
    "scan output left in fp32": (R, keep_f32, R),
    "generated tensors left in fp32": (keep_f32, R, R),
}


def _setup(shape):
    B, C, Cp, H, W, groups, cpw = shape
    inp = BlockInputs(B, C, Cp, H, W, rows=oracle.block_rows(Cp, 15, cpw), dirs=15, groups=groups,
                      cpw=cpw, dtype="bf16", seed=sum(shape))
    x, w_in, w_out = inp.f64()
    zhat = oracle.block_fwd(x, w_in, w_out, dirs=15, groups=groups, cpw=cpw, io_round=R)
    z, y = stand_in(inp, x, w_in, w_out, R, R, R)
    return inp, x, w_in, w_out, zhat, z, np.abs(y)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_rounding_block_passes(shape):
    inp, x, w_in, w_out, zhat, z, y_abs = _setup(shape)
    err = block_error(z, zhat, w_out, y_abs, "bf16")
    assert block_passes(err, "bf16"), err
    # with margin: the L2 residual of a correct block is well inside its bound
    assert err["l2"] < BLOCK_TOL["bf16"]["l2"] / 2, err


@pytest.mark.parametrize("mutant", sorted(MUTANTS))
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_misplaced_or_truncating_rounding_fails(shape, mutant):
    inp, x, w_in, w_out, zhat, _, y_abs = _setup(shape)
    z, _ = stand_in(inp, x, w_in, w_out, *MUTANTS[mutant])
    err = block_error(z, zhat, w_out, y_abs, "bf16")
    assert not block_passes(err, "bf16"), (mutant, err)
    # and with margin
    assert err["l2"] > 2 * BLOCK_TOL["bf16"]["l2"], (mutant, err)


def test_fp32_block_metric():
    # fp32 storage: the oracle is exact; an fp32 stand-in (no intermediate
    # rounding beyond fp32) passes, one whose scan output went through bf16
    # fails
    B, C, Cp, H, W, cpw = 2, 48, 16, 12, 10, 4
    inp = BlockInputs(B, C, Cp, H, W, rows=oracle.block_rows(Cp, 15, cpw), dirs=15, cpw=cpw, dtype="f32",
                      seed=4)
    x, w_in, w_out = inp.f64()
    zhat = oracle.block_fwd(x, w_in, w_out, dirs=15, cpw=cpw)
    z, y = stand_in(inp, x, w_in, w_out, keep_f32, keep_f32, keep_f32)
    assert block_passes(block_error(z, zhat, w_out, np.abs(y), "f32"), "f32")
    zb, _ = stand_in(inp, x, w_in, w_out, keep_f32, R, keep_f32)
    assert not block_passes(block_error(zb, zhat, w_out, np.abs(y), "f32"), "f32")


def test_non_finite_output_fails():
    inp, x, w_in, w_out, zhat, z, y_abs = _setup(SHAPES[0])
    z = z.copy()
    z[0, 0, 0, 0] = np.nan
    assert not block_passes(block_error(z, zhat, w_out, y_abs, "bf16"), "bf16")
