"""GPU parity of the compressed block (gspn_block_fwd) against the fp64 oracle.

The block is z = w_out . scan(x_proxy, taps, lambda, u) with x_proxy, taps,
lambda and u projected from x by w_in (oracle.block_fwd states the reading).

Metric (tests/parity.py, block_error): r_i = |z_i - zhat_i|, less the half
ulp of z_i's own bf16 rounding for bf16 I/O;
    pointwise = max_i r_i / s_i,   s_i = (|w_out| |y|)_i
(the sum of the magnitudes of the terms the output projection adds, floored
at 0.1 of its rms), and l2 = ||r|| / ||zhat||.

- fp32 I/O: the oracle is exact; the GEMMs accumulate in fp32 (about
  K 2^-24 relative with K <= 1152) and the scan meets its own 1e-4, so
  pointwise <= 2e-4 and l2 <= 2e-5.
- bf16 I/O: the block stores x_proxy, taps, lambda, u and y in bf16 and the
  oracle rounds the same tensors (oracle.round_bf16).  pointwise <= 2e-3
  (the scan's bf16 bound) and l2 <= 3e-4: a correct block differs only where
  an intermediate's fp32 and fp64 values round to neighbouring bf16 numbers,
  while a truncating or misplaced rounding moves every intermediate and puts
  l2 above 1e-3 (tests/test_block_metric.py plants those mistakes).
"""
import numpy as np
import pytest

import oracle
from parity import BLOCK_TOL, block_error, block_passes, from_device, say, to_device
from linear_spatial_propagation_amd.inputs import BLOCK_CONFIGS, BlockInputs

pytestmark = pytest.mark.gpu

def run_block(inp, out_batches=None, norm=True):
    import torch
    import linear_spatial_propagation_amd as gspn
    x, wi, wo = (to_device(a, inp.dtype) for a in (inp.x_store, inp.w_in_store, inp.w_out_store))
    z = gspn.block_fwd(x, wi, wo, dirs=inp.dirs, groups=inp.groups, ch_per_weight=inp.cpw, norm=norm)
    torch.cuda.synchronize()
    if out_batches is not None:
        z = z[out_batches]
    return from_device(z.contiguous(), inp.dtype)


def oracle_block(inp, batches=None, norm=True):
    x, wi, wo = inp.f64()
    if batches is not None:
        x = x[batches]
    rnd = oracle.round_bf16 if inp.dtype == "bf16" else None
    z = oracle.block_fwd(x, wi, wo, dirs=inp.dirs, groups=inp.groups, cpw=inp.cpw, norm=norm, io_round=rnd)
    return z, wo


CASES = [
    # B, C, C_proxy, H, W, dirs, groups, cpw
    (2, 24, 8, 16, 20, 15, 1, 2),     # fused scan
    (1, 40, 8, 64, 64, 15, 1, 8),     # one weight set for the proxy
    (2, 16, 4, 72, 40, 15, 2, 1),     # line kernels, local groups
    (1, 20, 6, 9, 7, 5, 1, 3),        # TB and LR, ragged sides
    (3, 8, 16, 12, 12, 15, 4, 4),     # proxy wider than the input
    (2, 64, 32, 16, 16, 15, 1, 4),
    (1, 96, 64, 24, 40, 15, 1, 8),
    (2, 160, 128, 8, 16, 15, 2, 16),  # the proxy width of the 1K block
    # the hand-written output projection (bf16): C_proxy in {16, ..., 256},
    # C % 32 == 0, H*W % 8 == 0, a partial last tile of 128 pixels
    (1, 32, 16, 9, 8, 15, 1, 4),
    (2, 64, 256, 12, 20, 15, 1, 32),
    (1, 96, 64, 17, 24, 3, 1, 8),
]


@pytest.mark.parametrize("norm", [True, False], ids=["rmsnorm", "plain"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_block_parity(case, dtype, norm):
    B, C, Cp, H, W, dirs, groups, cpw = case
    inp = BlockInputs(B, C, Cp, H, W, rows=oracle.block_rows(Cp, dirs, cpw), dirs=dirs, groups=groups,
                      cpw=cpw, dtype=dtype, seed=sum(case))
    say(f"block {case} {dtype} norm={norm}")
    z = run_block(inp, norm=norm)
    zhat, wo = oracle_block(inp, norm=norm)
    rnd = oracle.round_bf16 if dtype == "bf16" else None
    x, wi, _ = inp.f64()
    y = _scan_out(inp, x, wi, rnd, norm)
    err = block_error(z, zhat, wo, np.abs(y), dtype)
    say(f"  pointwise {err['pointwise']:.3e} l2 {err['l2']:.3e} (tol {BLOCK_TOL[dtype]})")
    assert block_passes(err, dtype), err


def _scan_out(inp, x, wi, rnd, norm=True):
    """The (normalised) scan output inside the oracle's block, the operand of
    the output projection (for the metric's scale)."""
    B, C, H, W = x.shape
    Cp, nd, Cw = inp.C_proxy, bin(inp.dirs).count("1"), inp.C_proxy // inp.cpw
    r = rnd or (lambda a: a)
    g = np.matmul(wi, x.reshape(B, C, H * W))
    t0, t1 = Cp, Cp + nd * Cw * 3
    taps = r(g[:, t0:t1]).reshape(B, nd, Cw, 3, H, W).transpose(1, 0, 2, 3, 4, 5)
    y = r(oracle.scan_fwd(r(g[:, :Cp]).reshape(B, Cp, H, W), taps, r(g[:, t1:t1 + Cp]).reshape(B, Cp, H, W),
                          r(g[:, t1 + Cp:]).reshape(B, Cp, H, W), dirs=inp.dirs, groups=inp.groups, cpw=inp.cpw))
    if norm:
        y = y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + oracle.BLOCK_NORM_EPS)
    return y


def test_block1k_sampled_batches():
    # the full 1K block (batch 32, C = 1152, C_proxy = 128, 64 x 64) runs
    # whole on the GPU; the oracle recomputes batch items 0 and 31
    cfg = dict(BLOCK_CONFIGS["block1k"])
    seed = cfg.pop("seed")
    inp = BlockInputs(cfg.pop("B"), cfg.pop("C"), cfg.pop("C_proxy"), cfg.pop("H"), cfg.pop("W"),
                      rows=oracle.block_rows(128, 15, cfg["cpw"]), seed=seed, **cfg)
    say("block1k, batches 0 and 31")
    sel = [0, inp.B - 1]
    z = run_block(inp, out_batches=sel)
    zhat, wo = oracle_block(inp, batches=sel)
    x, wi, _ = inp.f64()
    y = _scan_out(inp, x[sel], wi, oracle.round_bf16)
    err = block_error(z, zhat, wo, np.abs(y), "bf16")
    say(f"  pointwise {err['pointwise']:.3e} l2 {err['l2']:.3e} (tol {BLOCK_TOL['bf16']})")
    assert block_passes(err, "bf16"), err


def test_block_rejects_bad_weights():
    import torch
    import linear_spatial_propagation_amd as gspn
    x = torch.zeros(1, 8, 4, 4, device="cuda")
    with pytest.raises(ValueError):
        gspn.block_fwd(x, torch.zeros(10, 8, device="cuda"), torch.zeros(8, 4, device="cuda"))
