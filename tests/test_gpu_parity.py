"""GPU parity: the HIP library against the fp64 oracle, element by element.

Every call goes through the C ABI (libgspn.so via ctypes).  Small and
medium workloads are compared on every output; the two largest workloads
are compared on seeded sampled slices that the oracle computes one by one,
in the same launch configuration as the benchmark (the whole tensor is
computed on the GPU).
"""
import numpy as np
import pytest

import oracle
from parity import TOL, diagnostics, from_device, parity_error, run_workload, say, to_device
from linear_spatial_propagation_amd.inputs import (CONFIGS, config_workload, make_workload,
                                                   slice_inputs_f64)

pytestmark = pytest.mark.gpu

PATHS = {"auto": 0, "fused": 1, "general": 2, "slice": 3}


def check(wl, path="auto", tol=None):
    say(f"case B={wl.B} C={wl.C} H={wl.H} W={wl.W} dirs={wl.dirs} g={wl.groups} "
        f"cpw={wl.cpw} {wl.dtype} path={path}")
    y = run_workload(wl, PATHS[path])
    yhat = oracle.scan_fwd(wl.x, wl.w, wl.lam, wl.u, dirs=wl.dirs, groups=wl.groups, cpw=wl.cpw)
    err = parity_error(y, yhat, wl.dtype)
    diag = diagnostics(y, yhat, wl.dtype)
    say(f"  err={err:.3e}  " + " ".join(f"{k}={v:.3e}" for k, v in diag.items()))
    assert err <= (tol or TOL[wl.dtype]), err
    return y, yhat


# ------------------------------------------------------------ the workloads
@pytest.mark.parametrize("name", ["tiny", "cls56", "cgspn1k"])
def test_config_full_tensor(name):
    check(config_workload(name))


@pytest.mark.parametrize("name", ["tiny", "cgspn1k"])
def test_config_full_tensor_general_path(name):
    check(config_workload(name), path="general")


def sampled_slices(B, C, cpw, n, seed):
    rng = np.random.default_rng(seed)
    picks = {(0, 0), (B - 1, C - 1), (0, C - 1), (B - 1, 0)}
    if cpw > 1:
        picks |= {(0, cpw - 1), (0, cpw)}
    while len(picks) < n:
        picks.add((int(rng.integers(B)), int(rng.integers(C))))
    return sorted(picks)


@pytest.mark.parametrize("name,nslices", [("local2k", 64), ("hires512", 64)])
def test_config_sampled_slices(name, nslices):
    cfg = CONFIGS[name]
    say(f"case {name}: generating")
    wl = config_workload(name)
    say(f"case {name}: GPU")
    y = run_workload(wl)
    errs = []
    for (b, c) in sampled_slices(wl.B, wl.C, wl.cpw, nslices, 99):
        x, w, lam, u = slice_inputs_f64(cfg["seed"], b, c, H=wl.H, W=wl.W, dirs=wl.dirs,
                                        cpw=wl.cpw, dtype=wl.dtype, u_ones=cfg["u_ones"])
        yhat = oracle.slice_fwd(x, w, lam, u, dirs=wl.dirs, groups=wl.groups)
        errs.append(parity_error(y[b, c], yhat, wl.dtype))
    say(f"  max err over {len(errs)} slices = {max(errs):.3e}")
    assert max(errs) <= TOL[wl.dtype]


# Line path with channel-shared weights on launches large enough that each
# wave scans two channels of one weight set (the halved launch still has at
# least 8 waves per SIMD): one normalisation per pixel serves both.
LINE_SHARED = [
    # (B, C, H, W, dirs, groups, cpw, dtype)
    (4, 1024, 72, 72, 15, 1, 2, "bf16"),     # 2 positions per lane
    (4, 1024, 72, 72, 15, 4, 4, "bf16"),     # local groups
    (2, 2048, 132, 68, 15, 2, 4, "f32"),     # 4 positions per lane, fp32
]


@pytest.mark.parametrize("case", LINE_SHARED, ids=lambda c: "x".join(map(str, c)))
def test_line_path_channel_pairs_sampled_slices(case):
    B, C, H, W, dirs, g, cpw, dt = case
    seed = 40 + H + cpw
    say(f"case line pairs {case}: generating")
    wl = make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype=dt, seed=seed)
    say(f"case line pairs {case}: GPU")
    y = run_workload(wl, PATHS["general"])
    errs = []
    for (b, c) in sampled_slices(B, C, cpw, 24, seed):
        x, w, lam, u = slice_inputs_f64(seed, b, c, H=H, W=W, dirs=dirs, cpw=cpw, dtype=dt)
        errs.append(parity_error(y[b, c], oracle.slice_fwd(x, w, lam, u, dirs=dirs, groups=g), dt))
    say(f"  max err over {len(errs)} slices = {max(errs):.3e}")
    assert max(errs) <= TOL[dt]


# ------------------------------------------------------------ edge shapes
EDGE = [
    # (B, C, H, W, dirs, groups, cpw)
    (1, 2, 1, 1, 15, 1, 1),
    (1, 2, 1, 7, 15, 1, 1),
    (2, 3, 7, 1, 15, 1, 1),
    (1, 2, 2, 2, 15, 1, 2),
    (2, 4, 63, 63, 15, 1, 2),
    (1, 2, 64, 63, 15, 1, 1),
    (1, 2, 63, 64, 15, 1, 1),
    (2, 2, 56, 56, 15, 1, 1),
    (1, 3, 17, 45, 15, 1, 3),
    (1, 2, 64, 64, 15, 8, 1),
    (1, 2, 64, 64, 15, 64, 1),
    (1, 2, 32, 48, 15, 16, 2),
    (1, 4, 20, 30, 1, 1, 1),
    (1, 4, 20, 30, 2, 1, 1),
    (1, 4, 20, 30, 4, 1, 1),
    (1, 4, 20, 30, 8, 1, 1),
    (1, 4, 20, 30, 5, 1, 2),
    (1, 4, 20, 30, 10, 1, 4),
    (1, 4, 21, 31, 3, 1, 1),
    (1, 4, 21, 31, 12, 1, 1),
    (1, 4, 64, 64, 7, 2, 4),
    (3, 16, 64, 64, 15, 1, 16),   # one map shared by every channel
    (1, 128, 16, 16, 15, 1, 128), # few weight sets: channel chunks
    (2, 6, 8, 8, 15, 1, 3),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", EDGE, ids=lambda c: "x".join(map(str, c)))
def test_edge_shapes_fused(case, dtype):
    B, C, H, W, dirs, g, cpw = case
    check(make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype=dtype, seed=sum(case)))


EDGE_GENERAL = EDGE[:8] + [
    # line kernels: K = 2, 4, 8 positions per lane, direction subsets, groups
    (1, 2, 200, 136, 15, 1, 1),   # K = 4
    (1, 2, 256, 32, 15, 8, 2),    # K = 4, local groups, shared weights
    (1, 1, 320, 8, 15, 1, 1),     # K = 8, a very short side
    (2, 2, 96, 128, 3, 1, 1),     # row directions only: no transposes
    (2, 2, 128, 96, 12, 1, 1),    # column directions only
    (1, 3, 128, 64, 6, 4, 3),     # BT + LR, groups, cpw 3
    (1, 2, 512, 504, 15, 1, 1),   # K = 8, partial merge tiles
    # per-line fallback
    (1, 2, 65, 65, 15, 1, 1),
    (1, 2, 100, 37, 15, 1, 1),
    (1, 2, 1, 300, 15, 1, 1),
    (1, 2, 300, 2, 15, 1, 1),
    (1, 2, 128, 128, 15, 8, 1),
    (1, 2, 257, 65, 15, 1, 2),
    (1, 1, 600, 33, 9, 3, 1),
    (2, 4, 96, 80, 15, 16, 2),
    # the largest accepted side (GSPN_MAX_SIDE = 4096)
    (1, 1, 4096, 8, 15, 1, 1),
    (1, 1, 8, 4096, 12, 64, 1),
]


def test_maximum_grid():
    """4096 x 4096, the largest grid the ABI accepts, on the per-line fallback."""
    check(make_workload(1, 1, 4096, 4096, dtype="f32", seed=77), path="general")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", EDGE_GENERAL, ids=lambda c: "x".join(map(str, c)))
def test_edge_shapes_general(case, dtype):
    B, C, H, W, dirs, g, cpw = case
    check(make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype=dtype, seed=sum(case) + 1),
          path="general")


def test_fused_and_line_paths_agree_to_fp32_rounding():
    # the fused kernel and the line kernels sum in different orders, so their
    # fp32 results may differ in the last bits; each meets the oracle bound,
    # and they agree with each other within a few fp32 roundings of the
    # accumulated state (64 lines, about 64 * 2^-24 relative)
    wl = make_workload(2, 8, 40, 40, cpw=2, dtype="f32", seed=5)
    y1 = run_workload(wl, PATHS["fused"])
    y2 = run_workload(wl, PATHS["general"])
    yhat = oracle.scan_fwd(wl.x, wl.w, wl.lam, wl.u, cpw=2)
    assert parity_error(y1, yhat, "f32") <= 1e-4
    assert parity_error(y2, yhat, "f32") <= 1e-4
    scale = np.maximum(np.abs(yhat), 0.1 * np.sqrt(np.mean(yhat ** 2)))
    between = float((np.abs(y1 - y2) / scale).max())
    say(f"  fused vs line kernels: {between:.3e}")
    assert between <= 64 * 2.0 ** -24 * 4


# ------------------------------------------------------------ slice kernel
# one workgroup per (b, c) slice, the sum of the directions in LDS (bf16,
# H, W <= 128, W % 8 == 0, H even, groups >= 8, (W / groups) % 8 == 0 with
# LR or RL)
EDGE_SLICE = [
    # (B, C, H, W, dirs, groups, cpw)
    (1, 4, 128, 128, 15, 8, 1),     # the 2K local workload's slices
    (2, 3, 96, 64, 15, 8, 3),       # 12-line row groups, shared weights
    (1, 2, 128, 128, 15, 16, 1),    # two groups per wave; 8-column groups: LR with RL writing the output
    (1, 2, 128, 128, 3, 32, 2),     # row directions only, 4-line groups
    (1, 2, 72, 128, 12, 8, 1),      # column directions only, idle lanes
    (1, 2, 48, 64, 15, 8, 1),       # 6-line row groups, 8-line column groups
    (1, 2, 128, 64, 9, 8, 1),       # TB and RL
    (2, 2, 16, 64, 6, 8, 2),        # BT and LR, 2-line row groups
    (1, 3, 32, 64, 15, 8, 1),       # 4-line row groups, 8-column groups
    (1, 2, 120, 128, 15, 8, 2),     # 15-line row groups
    (1, 2, 128, 64, 3, 8, 1),       # TB then BT over 16-row groups, no column direction
    (2, 2, 128, 128, 7, 8, 2),      # TB, BT, then LR alone over 16-column groups
    (1, 2, 64, 128, 13, 4 * 2, 1),  # TB, then LR with RL writing the output
    (1, 2, 64, 64, 12, 8, 1),       # LR first then RL over 8-column groups
    (1, 2, 32, 128, 8, 8, 1),       # RL alone
    (1, 2, 128, 128, 4, 16, 1),     # LR alone, 8-column groups
    (1, 2, 64, 128, 9, 16, 1),      # TB, then RL alone over 8-column groups
    (2, 2, 64, 64, 13, 8, 2),       # TB, then LR with RL over 8-column groups
    (1, 2, 96, 128, 12, 16, 1),     # LR first with RL over 8-column groups
]


@pytest.mark.parametrize("case", EDGE_SLICE, ids=lambda c: "x".join(map(str, c)))
def test_edge_shapes_slice(case):
    B, C, H, W, dirs, g, cpw = case
    check(make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype="bf16", seed=sum(case) + 2),
          path="slice")


def test_slice_path_extreme_raw_taps():
    # raw taps spread over +-250: rows whose taps fall below -40 take the
    # exact-form normalisation
    wl = make_workload(1, 4, 128, 128, groups=8, dtype="bf16", seed=91)
    from linear_spatial_propagation_amd.inputs import bf16_round_bits, bf16_bits_to_f32
    w = bf16_bits_to_f32(wl.w_store) * np.float32(60.0)
    w[:, :, :, 1] -= np.float32(120.0)     # whole rows of very negative taps
    wl.w_store = bf16_round_bits(w)
    check(wl, path="slice")


def test_slice_path_rejects_unsupported_shapes():
    import torch
    from linear_spatial_propagation_amd import _lib
    x = torch.zeros((1, 2, 128, 128), dtype=torch.float32, device="cuda")
    w = torch.zeros((4, 1, 2, 3, 128, 128), dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    # fp32, and too few groups
    assert _lib.scan_fwd_ptr(x.data_ptr(), w.data_ptr(), x.data_ptr(), x.data_ptr(), y.data_ptr(), 1, 2, 128, 128,
                             groups=8, dtype=_lib.GSPN_F32, path=3) == -10
    xb = x.to(torch.bfloat16)
    wb = w.to(torch.bfloat16)
    yb = torch.empty_like(xb)
    assert _lib.scan_fwd_ptr(xb.data_ptr(), wb.data_ptr(), xb.data_ptr(), xb.data_ptr(), yb.data_ptr(), 1, 2, 128,
                             128, groups=4, path=3) == -10
