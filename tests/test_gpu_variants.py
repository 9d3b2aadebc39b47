"""GPU parity of the per-direction variant (gspn_scan_fwd_ex): per-direction
lambda and/or u, checked against the oracle's variant element by element
with the forward's metric and tolerances.  Also the fully shared weight map
(ch_per_weight = C, GSPN-2's single map) on the default entry point."""
import numpy as np
import pytest

import oracle
from parity import TOL, from_device, parity_error, say, to_device
from linear_spatial_propagation_amd.inputs import make_workload, _store, bf16_bits_to_f32

pytestmark = pytest.mark.gpu


def per_dir(wl, seed, what):
    """Seeded per-direction slabs [nd][B][C][H][W] in the workload's dtype
    (lambda ~ U(0, 1), u ~ U(0, 1)), as stored and as fp64."""
    nd = bin(wl.dirs).count("1")
    rng = np.random.default_rng([seed, 3 if what == "lam" else 4])
    a32 = rng.random((nd, wl.B, wl.C, wl.H, wl.W), dtype=np.float32)
    st = _store(a32, wl.dtype)
    f64 = bf16_bits_to_f32(st).astype(np.float64) if wl.dtype == "bf16" else st.astype(np.float64)
    return st, f64


def check(case, dtype, lam_dir, u_dir):
    import torch
    import linear_spatial_propagation_amd as gspn
    B, C, H, W, dirs, g, cpw = case
    seed = sum(case) + 11
    wl = make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype=dtype, seed=seed)
    lam_st, lam64 = per_dir(wl, seed, "lam") if lam_dir else (wl.lam_store, wl.lam)
    u_st, u64 = per_dir(wl, seed, "u") if u_dir else (wl.u_store, wl.u)
    say(f"case variant B={B} C={C} H={H} W={W} dirs={dirs} g={g} cpw={cpw} {dtype} "
        f"lam_dir={lam_dir} u_dir={u_dir}")
    y = gspn.scan_fwd_dirs(to_device(wl.x_store, dtype), to_device(wl.w_store, dtype),
                           to_device(lam_st, dtype), to_device(u_st, dtype), dirs=dirs, groups=g,
                           ch_per_weight=cpw)
    torch.cuda.synchronize()
    yhat = oracle.scan_fwd_dirs(wl.x, wl.w, lam64, u64, dirs=dirs, groups=g, cpw=cpw)
    err = parity_error(from_device(y, dtype), yhat, dtype)
    say(f"  err={err:.3e}")
    assert err <= TOL[dtype], err


CASES = [
    (2, 16, 64, 64, 15, 1, 8),    # the 1K C-GSPN shape at small B
    (2, 4, 56, 56, 15, 1, 1),
    (1, 4, 20, 30, 15, 2, 2),     # whole-grid edge tiles, groups
    (1, 2, 200, 136, 15, 1, 1),   # K = 4
    (1, 4, 128, 96, 12, 1, 4),    # column directions only
    (1, 4, 96, 128, 3, 1, 2),     # row directions only
    (1, 3, 128, 64, 6, 4, 3),     # BT + LR
    (1, 2, 33, 17, 9, 1, 1),      # TB + RL, ragged tiles
]


@pytest.mark.parametrize("flags", [(True, False), (False, True), (True, True)], ids=["lam", "u", "both"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_variant_parity(case, dtype, flags):
    check(case, dtype, *flags)


def test_variant_replicated_slabs_equal_shared_call():
    """Per-direction tensors that repeat one slab give gspn_scan_fwd's result."""
    import torch
    import linear_spatial_propagation_amd as gspn
    wl = make_workload(2, 8, 48, 40, cpw=2, dtype="f32", seed=21)
    dev = [to_device(a, "f32") for a in (wl.x_store, wl.w_store, wl.lam_store, wl.u_store)]
    y_shared = gspn.scan_fwd(*dev, ch_per_weight=2, path=gspn.PATH_GENERAL)
    rep = lambda t: t.unsqueeze(0).repeat(4, 1, 1, 1, 1).contiguous()
    y_dir = gspn.scan_fwd_dirs(dev[0], dev[1], rep(dev[2]), rep(dev[3]), ch_per_weight=2)
    torch.cuda.synchronize()
    # the same scans; only the merge's rounding order differs
    np.testing.assert_allclose(y_dir.cpu().numpy(), y_shared.cpu().numpy(), rtol=1e-5, atol=1e-5)


# ------------------------------------------------------------ backward of the variant
def check_bwd(case, dtype, lam_dir, u_dir):
    import torch
    import linear_spatial_propagation_amd as gspn
    from linear_spatial_propagation_amd.inputs import gy_f64, make_gy
    B, C, H, W, dirs, g, cpw = case
    seed = sum(case) + 23
    wl = make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype=dtype, seed=seed)
    lam_st, lam64 = per_dir(wl, seed, "lam") if lam_dir else (wl.lam_store, wl.lam)
    u_st, u64 = per_dir(wl, seed, "u") if u_dir else (wl.u_store, wl.u)
    gy = make_gy(wl, seed + 1)
    say(f"case variant bwd B={B} C={C} H={H} W={W} dirs={dirs} g={g} cpw={cpw} {dtype} "
        f"lam_dir={lam_dir} u_dir={u_dir}")
    got = gspn.scan_bwd_dirs(*(to_device(a, dtype) for a in (wl.x_store, wl.w_store, lam_st, u_st, gy)),
                             dirs=dirs, groups=g, ch_per_weight=cpw)
    torch.cuda.synchronize()
    want = oracle.scan_bwd_dirs(wl.x, wl.w, lam64, u64, gy_f64(gy, dtype), dirs=dirs, groups=g, cpw=cpw)
    errs = {nm: parity_error(from_device(t, dtype), w, dtype)
            for nm, t, w in zip(("gx", "gw", "glam", "gu"), got, want)}
    say("  " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("flags", [(True, False), (False, True), (True, True)], ids=["lam", "u", "both"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_variant_bwd_parity(case, dtype, flags):
    check_bwd(case, dtype, *flags)


def test_variant_bwd_replicated_slabs_equal_shared_call():
    """Per-direction slabs that repeat one tensor: gx and gw equal gspn_scan_bwd's,
    the per-slab glam and gu sum to its glam and gu."""
    import torch
    import linear_spatial_propagation_amd as gspn
    from linear_spatial_propagation_amd.inputs import make_gy
    wl = make_workload(2, 8, 48, 40, cpw=2, dtype="f32", seed=22)
    dev = [to_device(a, "f32") for a in (wl.x_store, wl.w_store, wl.lam_store, wl.u_store, make_gy(wl, 5))]
    shared = gspn.scan_bwd(*dev, ch_per_weight=2, path=gspn.PATH_GENERAL)
    rep = lambda t: t.unsqueeze(0).repeat(4, 1, 1, 1, 1).contiguous()
    gx, gw, glam, gu = gspn.scan_bwd_dirs(dev[0], dev[1], rep(dev[2]), rep(dev[3]), dev[4], ch_per_weight=2)
    torch.cuda.synchronize()
    for got, want in ((gx, shared[0]), (gw, shared[1]), (glam.sum(0), shared[2]), (gu.sum(0), shared[3])):
        np.testing.assert_allclose(got.cpu().numpy(), want.cpu().numpy(), rtol=1e-5, atol=1e-5)
