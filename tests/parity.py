"""Shared helpers of the GPU parity tests: upload, run, compare.

The comparison metric.  For every output element i, with the oracle value
yhat_i (fp64) and the device value y_i widened to fp64:

    r_i   = |y_i - yhat_i|                                   (fp32 I/O)
    r_i   = max(0, |y_i - yhat_i| - ulp_bf16(y_i) / 2)       (bf16 I/O)
    err   = max_i  r_i / max(|yhat_i|, 0.1 * rms(yhat))

For bf16 I/O the final rounding of y to bf16 is exact-by-definition (the
half-ulp is subtracted), so err measures the fp32 accumulation error of the
path; the floor 0.1 * rms keeps outputs that cancel to ~0 from dividing by
~0.  Tolerances: err <= 1e-4 for fp32 I/O, err <= 2e-3 for bf16 I/O, and no
NaN or Inf anywhere.
"""
from __future__ import annotations

import sys

import numpy as np

from linear_spatial_propagation_amd.inputs import bf16_bits_to_f32

TOL = {"f32": 1e-4, "bf16": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def ulp_bf16(y: np.ndarray) -> np.ndarray:
    m, e = np.frexp(np.abs(y))            # |y| = m * 2^e, m in [0.5, 1)
    return np.where(y == 0, 0.0, np.ldexp(1.0, e - 8))


def parity_error(y: np.ndarray, yhat: np.ndarray, dtype: str) -> float:
    y = np.asarray(y, dtype=np.float64)
    yhat = np.asarray(yhat, dtype=np.float64)
    if y.shape != yhat.shape:
        raise AssertionError(f"shape {y.shape} != {yhat.shape}")
    if not np.all(np.isfinite(y)):
        return float("inf")
    diff = np.abs(y - yhat)
    if dtype == "bf16":
        diff = np.maximum(0.0, diff - 0.5 * ulp_bf16(y))
    rms = float(np.sqrt(np.mean(yhat * yhat))) if yhat.size else 0.0
    scale = np.maximum(np.abs(yhat), 0.1 * rms)
    scale = np.where(scale == 0, 1.0, scale)
    return float((diff / scale).max()) if y.size else 0.0


def rne_bf16(yhat: np.ndarray) -> np.ndarray:
    """fp64 values rounded once to the nearest bf16 (ties to even), as fp64."""
    yhat = np.asarray(yhat, dtype=np.float64)
    ulp = ulp_bf16(yhat)
    safe = np.where(ulp == 0, 1.0, ulp)
    return np.where(ulp == 0, 0.0, np.round(yhat / safe) * safe)   # np.round: half to even


def diagnostics(y: np.ndarray, yhat: np.ndarray, dtype: str) -> dict:
    """Side figures of a comparison (reported, not asserted): the unfloored
    pointwise maximum relative error, the L2-relative error and, for bf16,
    the fraction of outputs that differ from the correctly rounded exact value."""
    y = np.asarray(y, dtype=np.float64)
    yhat = np.asarray(yhat, dtype=np.float64)
    nz = yhat != 0
    out = {
        "pointwise_max": float((np.abs(y - yhat)[nz] / np.abs(yhat[nz])).max()) if nz.any() else 0.0,
        "l2_rel": float(np.linalg.norm(y - yhat) / max(np.linalg.norm(yhat), 1e-300)),
    }
    if dtype == "bf16":
        out["frac_not_rne"] = float(np.mean(y != rne_bf16(yhat)))
    return out


def to_device(a: np.ndarray, dtype: str):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype == "bf16":
        t = t.view(torch.bfloat16)
    return t.cuda()


def from_device(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def run_workload(wl, path: int = 0):
    """Upload a Workload, run the HIP scan, return y as fp64 numpy."""
    import torch
    import linear_spatial_propagation_amd as gspn
    x = to_device(wl.x_store, wl.dtype)
    w = to_device(wl.w_store, wl.dtype)
    lam = to_device(wl.lam_store, wl.dtype)
    u = to_device(wl.u_store, wl.dtype)
    y = gspn.scan_fwd(x, w, lam, u, dirs=wl.dirs, groups=wl.groups, ch_per_weight=wl.cpw, path=path)
    torch.cuda.synchronize()
    return from_device(y, wl.dtype)


# ------------------------------------------------------------------ block
# Tolerances of the compressed block (projection, scan, projection back).
#  pointwise: the scan's own bound (1e-4 fp32, 2e-3 bf16) on the scale of the
#             output projection's terms; fp32 also carries the two GEMMs'
#             fp32 accumulation (about K 2^-24 relative with K <= 1152), so
#             2e-4 there.
#  l2:        the residual over all outputs.  In bf16 the block stores five
#             intermediates rounded to nearest even, and the oracle rounds the
#             same five; what a correct block may still differ by is the rare
#             intermediate whose fp32 and fp64 values round to neighbouring
#             bf16 numbers (one ulp, 2^-8 relative, on under 1% of them).  A
#             store that truncates, or a rounding at another place, moves every
#             intermediate instead: 2^-9 relative on average, which puts the L2
#             residual above 1e-3.  The bound 3e-4 sits between the two.
BLOCK_TOL = {"f32": {"pointwise": 2e-4, "l2": 2e-5}, "bf16": {"pointwise": 2e-3, "l2": 3e-4}}


def block_error(z, zhat, w_out, y_abs, dtype: str) -> dict:
    """Parity figures of a block output z against the oracle's zhat.

    r_i = |z_i - zhat_i| (fp32 I/O), or max(0, |z_i - zhat_i| - ulp_bf16(z_i)/2)
    (bf16 I/O: the final rounding of z is exact by definition, as in the scan
    metric).  s_i = (|w_out| |y|)_i, the sum of the magnitudes of the terms
    the output projection adds at element i, floored at 0.1 of its rms.
      pointwise = max_i r_i / s_i
      l2        = ||r||_2 / ||zhat||_2
    Non-finite output scores inf on both."""
    z = np.asarray(z, dtype=np.float64)
    zhat = np.asarray(zhat, dtype=np.float64)
    if z.shape != zhat.shape:
        raise AssertionError(f"shape {z.shape} != {zhat.shape}")
    if not np.all(np.isfinite(z)):
        return {"pointwise": float("inf"), "l2": float("inf")}
    r = np.abs(z - zhat)
    if dtype == "bf16":
        r = np.maximum(0.0, r - 0.5 * ulp_bf16(z))
    s = np.einsum("cq,bqhw->bchw", np.abs(np.asarray(w_out, dtype=np.float64)), y_abs)
    s = np.maximum(s, 0.1 * float(np.sqrt(np.mean(s * s))))
    s = np.where(s == 0, 1.0, s)
    return {"pointwise": float((r / s).max()),
            "l2": float(np.linalg.norm(r) / max(float(np.linalg.norm(zhat)), 1e-300))}


def block_passes(err: dict, dtype: str) -> bool:
    tol = BLOCK_TOL[dtype]
    return err["pointwise"] <= tol["pointwise"] and err["l2"] <= tol["l2"]
