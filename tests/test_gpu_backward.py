"""GPU parity of the backward (gspn_scan_bwd) against the fp64 oracle.

All four gradients (gx, gw_raw, glam, gu) are compared element by element
with the metric of the forward parity tests (parity.py): err <= 1e-4 for
fp32 I/O and <= 2e-3 for bf16 I/O beyond the final rounding.  Small shapes
are compared on the whole tensor; the benchmark workloads are run whole on
the GPU and compared on sampled weight sets (b, k) -- every channel of a
sampled set, so that its tap gradients are complete -- which the oracle
computes one set at a time.  Every call goes through the C ABI.
"""
import numpy as np
import pytest

import oracle
from parity import TOL, from_device, parity_error, say, to_device
from linear_spatial_propagation_amd.inputs import (CONFIGS, config_workload, gy_f64, make_gy,
                                                   make_workload, slice_gy, slice_inputs_f64)

pytestmark = pytest.mark.gpu

NAMES = ("gx", "gw", "glam", "gu")


PATHS = {"auto": 0, "fused": 1, "lines": 2}


def run_bwd(wl, gy_store, path="auto"):
    import torch
    import linear_spatial_propagation_amd as gspn
    dev = [to_device(a, wl.dtype) for a in (wl.x_store, wl.w_store, wl.lam_store, wl.u_store, gy_store)]
    out = gspn.scan_bwd(*dev, dirs=wl.dirs, groups=wl.groups, ch_per_weight=wl.cpw, path=PATHS[path])
    torch.cuda.synchronize()
    return [from_device(t, wl.dtype) for t in out]


def errors(got, want, dtype):
    return {nm: parity_error(g, w, dtype) for nm, g, w in zip(NAMES, got, want)}


def check(wl, seed, path="auto"):
    say(f"case bwd B={wl.B} C={wl.C} H={wl.H} W={wl.W} dirs={wl.dirs} g={wl.groups} "
        f"cpw={wl.cpw} {wl.dtype} path={path}")
    gy = make_gy(wl, seed)
    got = run_bwd(wl, gy, path)
    want = oracle.scan_bwd(wl.x, wl.w, wl.lam, wl.u, gy_f64(gy, wl.dtype), dirs=wl.dirs,
                           groups=wl.groups, cpw=wl.cpw)
    errs = errors(got, want, wl.dtype)
    say("  " + " ".join(f"{k}={v:.3e}" for k, v in errs.items()))
    assert max(errs.values()) <= TOL[wl.dtype], errs


EDGE_BWD = [
    # (B, C, H, W, dirs, groups, cpw)
    (1, 2, 1, 1, 15, 1, 1),
    (1, 2, 1, 7, 15, 1, 1),       # lines of length 1 (LR, RL)
    (2, 3, 7, 1, 15, 1, 1),
    (1, 2, 2, 2, 15, 1, 2),
    (2, 4, 63, 63, 15, 1, 2),
    (1, 3, 17, 45, 15, 1, 3),     # three chunks of one channel
    (1, 2, 64, 64, 15, 8, 1),
    (1, 2, 64, 64, 15, 64, 1),    # every line starts a group
    (1, 2, 32, 48, 15, 16, 2),
    (1, 4, 20, 30, 1, 1, 1),
    (1, 4, 20, 30, 2, 1, 1),
    (1, 4, 20, 30, 4, 1, 1),
    (1, 4, 20, 30, 8, 1, 1),
    (1, 4, 20, 30, 5, 1, 2),
    (1, 4, 20, 30, 10, 1, 4),
    (1, 8, 24, 24, 15, 1, 8),     # one chunk of eight channels
    (1, 32, 16, 16, 15, 1, 16),   # two chunks of eight
    (1, 24, 16, 8, 15, 1, 24),    # three chunks of eight
    (1, 2, 200, 136, 15, 1, 1),   # K = 4
    (1, 4, 256, 32, 15, 8, 2),    # K = 4, groups, one chunk of two
    (1, 8, 128, 64, 15, 1, 8),    # K = 2, two chunks of four
    (1, 1, 320, 8, 15, 1, 1),     # K = 8
    (1, 4, 96, 128, 3, 1, 2),     # row directions only
    (1, 4, 128, 96, 12, 1, 4),    # column directions only
    (1, 3, 128, 64, 6, 4, 3),
    (1, 2, 512, 504, 15, 1, 2),   # K = 8, two chunks of one
    (1, 2, 264, 272, 15, 4, 1),   # K = 8 (lines held by two waves), local groups
    (1, 3, 512, 16, 15, 1, 3),    # K = 8, three chunks of one; row lines fit one wave
    (2, 1, 264, 264, 5, 1, 1),    # K = 8, TB and LR only
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", EDGE_BWD, ids=lambda c: "x".join(map(str, c)))
def test_bwd_edge_shapes(case, dtype):
    B, C, H, W, dirs, g, cpw = case
    seed = sum(case) + 7
    check(make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype=dtype, seed=seed), seed + 100)


# the line kernels on shapes that the fused kernel takes by default
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", [c for c in EDGE_BWD if max(c[2], c[3]) <= 64],
                         ids=lambda c: "x".join(map(str, c)))
def test_bwd_edge_shapes_line_kernels(case, dtype):
    B, C, H, W, dirs, g, cpw = case
    seed = sum(case) + 7
    check(make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype=dtype, seed=seed), seed + 100,
          path="lines")


def test_bwd_tiny_full():
    check(config_workload("tiny"), 11)


@pytest.mark.parametrize("path", ["fused", "lines"])
def test_bwd_cgspn1k_full(path):
    check(config_workload("cgspn1k"), 1002, path=path)


def sampled_sets(B, Cw, n, seed):
    rng = np.random.default_rng(seed)
    picks = {(0, 0), (B - 1, Cw - 1)}
    while len(picks) < min(n, B * Cw):
        picks.add((int(rng.integers(B)), int(rng.integers(Cw))))
    return sorted(picks)


@pytest.mark.parametrize("name,nsets", [("cls56", 24), ("cgspn1k", 12), ("local2k", 12),
                                        ("hires512", 4)])
def test_bwd_config_sampled_sets(name, nsets):
    cfg = CONFIGS[name]
    say(f"case bwd {name}: generating")
    wl = config_workload(name)
    gseed = 1000 + cfg["seed"]
    gy = make_gy(wl, gseed)
    say(f"case bwd {name}: GPU")
    got = run_bwd(wl, gy)
    cpw, Cw = wl.cpw, wl.C // wl.cpw
    worst = {nm: 0.0 for nm in NAMES}
    for (b, k) in sampled_sets(wl.B, Cw, nsets, 77):
        chans = range(k * cpw, (k + 1) * cpw)
        parts = [slice_inputs_f64(cfg["seed"], b, c, H=wl.H, W=wl.W, dirs=wl.dirs, cpw=cpw,
                                  dtype=wl.dtype, u_ones=cfg["u_ones"]) for c in chans]
        x = np.stack([p[0] for p in parts])[None]
        w = parts[0][1][:, None, None]                     # [nd][1][1][3][H][W]
        lam = np.stack([p[2] for p in parts])[None]
        u = np.stack([p[3] for p in parts])[None]
        g = np.stack([gy_f64(gy[b, c], wl.dtype) for c in chans])[None]
        want = oracle.scan_bwd(x, w, lam, u, g, dirs=wl.dirs, groups=wl.groups, cpw=cpw)
        have = (got[0][b, k * cpw:(k + 1) * cpw][None], got[1][:, b, k][:, None, None],
                got[2][b, k * cpw:(k + 1) * cpw][None], got[3][b, k * cpw:(k + 1) * cpw][None])
        for nm, v in errors(have, want, wl.dtype).items():
            worst[nm] = max(worst[nm], v)
    say("  worst " + " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    assert max(worst.values()) <= TOL[wl.dtype], worst


def test_bwd_line_path_channel_pairs_sampled_sets():
    # large enough that the line kernels' forward pass scans two channels of a
    # weight set per wave
    B, C, H, W, cpw, seed = 2, 2048, 72, 72, 2, 71
    say("case bwd line pairs: generating")
    wl = make_workload(B, C, H, W, groups=1, cpw=cpw, dtype="bf16", seed=seed)
    gy = make_gy(wl, seed + 1)
    say("case bwd line pairs: GPU")
    got = run_bwd(wl, gy)
    Cw = C // cpw
    worst = {nm: 0.0 for nm in NAMES}
    for (b, k) in sampled_sets(B, Cw, 6, 78):
        chans = range(k * cpw, (k + 1) * cpw)
        parts = [slice_inputs_f64(seed, b, c, H=H, W=W, dirs=15, cpw=cpw, dtype="bf16") for c in chans]
        x = np.stack([p[0] for p in parts])[None]
        w = parts[0][1][:, None, None]
        lam = np.stack([p[2] for p in parts])[None]
        u = np.stack([p[3] for p in parts])[None]
        g = np.stack([gy_f64(gy[b, c], "bf16") for c in chans])[None]
        want = oracle.scan_bwd(x, w, lam, u, g, dirs=15, groups=1, cpw=cpw)
        have = (got[0][b, k * cpw:(k + 1) * cpw][None], got[1][:, b, k][:, None, None],
                got[2][b, k * cpw:(k + 1) * cpw][None], got[3][b, k * cpw:(k + 1) * cpw][None])
        for nm, v in errors(have, want, "bf16").items():
            worst[nm] = max(worst[nm], v)
    say("  worst " + " ".join(f"{k}={v:.3e}" for k, v in worst.items()))
    assert max(worst.values()) <= TOL["bf16"], worst


@pytest.mark.parametrize("path", ["fused", "lines"])
@pytest.mark.parametrize("scale", [12.0, 60.0])
def test_bwd_wide_raw_taps(path, scale):
    """Raw taps far from 0 (sigmoids near 0 or 1; below -25 the fused kernel
    takes its exact per-tap form, below -40 the line kernels do)."""
    for (H, W, g) in [(20, 32, 2), (64, 64, 1)]:
        wl = make_workload(1, 4, H, W, groups=g, cpw=2, dtype="f32", seed=int(scale) + H)
        wl.w_store = (wl.w_store * np.float32(scale)).astype(np.float32)
        check(wl, 9, path=path)


def test_bwd_ones_invariant():
    """x = lam = u = 1: y is the same for every choice of taps (Theorem 1 of
    "Key design 1"), so the tap gradient is 0 and gu = gy * ((H/g+1) + (W/g+1))."""
    import torch
    import linear_spatial_propagation_amd as gspn
    B, C, H, W, g = 2, 16, 48, 40, 4
    torch.manual_seed(0)
    one = torch.ones(B, C, H, W, device="cuda")
    w = (3 * torch.randn(4, B, C // 2, 3, H, W)).cuda()
    gy = torch.randn(B, C, H, W).cuda()
    gx, gw, glam, gu = gspn.scan_bwd(one, w, one, one, gy, groups=g, ch_per_weight=2)
    torch.cuda.synchronize()
    scale = float(gy.abs().max()) * H * W
    assert float(gw.abs().max()) <= 1e-5 * scale
    np.testing.assert_allclose(gu.cpu().numpy(), (gy * ((H // g + 1) + (W // g + 1))).cpu().numpy(),
                               rtol=1e-6, atol=1e-5)
    np.testing.assert_array_equal(gx.cpu().numpy(), glam.cpu().numpy())


def test_bwd_unread_taps_are_ignored_and_get_zero():
    """NaN in taps the forward never reads changes nothing, and their gradient is exactly 0."""
    import torch
    import linear_spatial_propagation_amd as gspn
    wl = make_workload(1, 4, 24, 32, groups=4, cpw=2, dtype="f32", seed=3)
    gy = make_gy(wl, 5)
    clean = run_bwd(wl, gy)
    w = wl.w_store.copy()
    H, W, L_r, L_c = 24, 32, 6, 8
    w[0, :, :, :, ::L_r] = np.nan          # TB: first rows of groups
    w[1, :, :, :, L_r - 1::L_r] = np.nan   # BT
    w[2, :, :, :, :, ::L_c] = np.nan       # LR: first columns of groups
    w[3, :, :, :, :, L_c - 1::L_c] = np.nan
    w[0:2, :, :, 0, :, 0] = np.nan         # missing left / right neighbours
    w[0:2, :, :, 2, :, W - 1] = np.nan
    w[2:4, :, :, 0, 0, :] = np.nan
    w[2:4, :, :, 2, H - 1, :] = np.nan
    wl.w_store = w
    dirty = run_bwd(wl, gy)
    for a, b_ in zip(clean, dirty):
        np.testing.assert_array_equal(a, b_)
    gw = dirty[1]
    assert not gw[0, :, :, :, ::L_r].any() and not gw[2, :, :, :, :, ::L_c].any()
    assert not gw[0:2, :, :, 0, :, 0].any() and not gw[2:4, :, :, 2, H - 1, :].any()


def test_autograd_wrapper_gives_the_backward_gradients():
    """gspn_scan under autograd: the gradients of sum(y * gy) are exactly
    scan_bwd's outputs (the same kernels), and y is scan_fwd's."""
    import torch
    import linear_spatial_propagation_amd as gspn
    wl = make_workload(2, 8, 40, 48, groups=2, cpw=4, dtype="bf16", seed=61)
    gy = to_device(make_gy(wl, 62), "bf16")
    leaves = [to_device(a, "bf16").requires_grad_() for a in (wl.x_store, wl.w_store, wl.lam_store, wl.u_store)]
    y = gspn.gspn_scan(*leaves, groups=2, ch_per_weight=4)
    (y.float() * gy.float()).sum().backward()
    plain = [t.detach() for t in leaves]
    y_ref = gspn.scan_fwd(*plain, groups=2, ch_per_weight=4)
    want = gspn.scan_bwd(*plain, gy, groups=2, ch_per_weight=4)
    torch.cuda.synchronize()
    assert torch.equal(y.detach(), y_ref)
    for leaf, w in zip(leaves, want):
        assert torch.equal(leaf.grad, w)
