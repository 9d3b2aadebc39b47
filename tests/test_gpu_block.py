"""GPU parity of the compressed block (gspn_block_fwd) against the fp64 oracle.

The block is z = w_out . scan(x_proxy, taps, lambda, u) with x_proxy, taps,
lambda and u projected from x by w_in (oracle.block_fwd states the reading).

Metric: for every output element i, with the oracle value zhat_i,
    err = max_i |z_i - zhat_i| / s_i,   s_i = (|w_out| |y|)_i
the sum of the magnitudes of the terms the output projection adds (floored
at 0.1 of its rms), so that outputs that cancel are not divided by ~0.

- fp32 I/O: the oracle is exact.  The GEMMs accumulate in fp32 (relative
  error about K 2^-24 with K <= 1152, below 1e-4) and the scan meets its own
  1e-4 bound, so err <= 2e-4.
- bf16 I/O: the block stores x_proxy, taps, lambda, u and y in bf16, and the
  oracle rounds the same tensors (oracle.round_bf16).  What remains is the
  final rounding of z (half an ulp, 2^-9 relative), the scan's own 2e-3
  bound, and the rare intermediate whose fp32 GEMM sum and fp64 sum round to
  neighbouring bf16 values (one ulp, 2^-8 relative, at that element only):
  err <= 1e-2.
"""
import numpy as np
import pytest

import oracle
from parity import from_device, say, to_device
from linear_spatial_propagation_amd.inputs import BLOCK_CONFIGS, BlockInputs

pytestmark = pytest.mark.gpu

TOL = {"f32": 2e-4, "bf16": 1e-2}


def block_error(z, zhat, w_out, y_abs):
    s = np.einsum("cq,bqhw->bchw", np.abs(w_out), y_abs)
    rms = float(np.sqrt(np.mean(s * s)))
    s = np.maximum(s, 0.1 * rms)
    if not np.all(np.isfinite(z)):
        return float("inf")
    return float((np.abs(z - zhat) / s).max())


def run_block(inp, out_batches=None):
    import torch
    import linear_spatial_propagation_amd as gspn
    x, wi, wo = (to_device(a, inp.dtype) for a in (inp.x_store, inp.w_in_store, inp.w_out_store))
    z = gspn.block_fwd(x, wi, wo, dirs=inp.dirs, groups=inp.groups, ch_per_weight=inp.cpw)
    torch.cuda.synchronize()
    if out_batches is not None:
        z = z[out_batches]
    return from_device(z.contiguous(), inp.dtype)


def oracle_block(inp, batches=None):
    x, wi, wo = inp.f64()
    if batches is not None:
        x = x[batches]
    rnd = oracle.round_bf16 if inp.dtype == "bf16" else None
    z = oracle.block_fwd(x, wi, wo, dirs=inp.dirs, groups=inp.groups, cpw=inp.cpw, io_round=rnd)
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
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_block_parity(case, dtype):
    B, C, Cp, H, W, dirs, groups, cpw = case
    inp = BlockInputs(B, C, Cp, H, W, rows=oracle.block_rows(Cp, dirs, cpw), dirs=dirs, groups=groups,
                      cpw=cpw, dtype=dtype, seed=sum(case))
    say(f"block {case} {dtype}")
    z = run_block(inp)
    zhat, wo = oracle_block(inp)
    rnd = oracle.round_bf16 if dtype == "bf16" else None
    x, wi, _ = inp.f64()
    y = _scan_out(inp, x, wi, rnd)
    err = block_error(z, zhat, wo, np.abs(y))
    say(f"  err {err:.3e} (tol {TOL[dtype]:.0e})")
    assert err <= TOL[dtype]


def _scan_out(inp, x, wi, rnd):
    """The scan output inside the oracle's block (for the metric's scale)."""
    B, C, H, W = x.shape
    Cp, nd, Cw = inp.C_proxy, bin(inp.dirs).count("1"), inp.C_proxy // inp.cpw
    r = rnd or (lambda a: a)
    g = np.matmul(wi, x.reshape(B, C, H * W))
    t0, t1 = Cp, Cp + nd * Cw * 3
    taps = r(g[:, t0:t1]).reshape(B, nd, Cw, 3, H, W).transpose(1, 0, 2, 3, 4, 5)
    return oracle.scan_fwd(r(g[:, :Cp]).reshape(B, Cp, H, W), taps, r(g[:, t1:t1 + Cp]).reshape(B, Cp, H, W),
                           r(g[:, t1 + Cp:]).reshape(B, Cp, H, W), dirs=inp.dirs, groups=inp.groups, cpw=inp.cpw)


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
    err = block_error(z, zhat, wo, np.abs(y))
    say(f"  err {err:.3e} (tol {TOL['bf16']:.0e})")
    assert err <= TOL["bf16"]


def test_block_rejects_bad_weights():
    import torch
    import linear_spatial_propagation_amd as gspn
    x = torch.zeros(1, 8, 4, 4, device="cuda")
    with pytest.raises(ValueError):
        gspn.block_fwd(x, torch.zeros(10, 8, device="cuda"), torch.zeros(8, 4, device="cuda"))
