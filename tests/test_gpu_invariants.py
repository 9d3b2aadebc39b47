"""GPU checks that need no oracle: invariants and exact special cases.

These are independent evidence for the HIP path: the ones invariant
(Theorem 1 of "Key design 1: stability-context condition", GSPN CVPR 2025
paper notes), the g = n pointwise case ("Key design 3"), a hand-derived
example, determinism, ignored taps, extreme raw taps and stream ordering.
"""
import os

import numpy as np
import pytest

import oracle
from parity import TOL, from_device, parity_error, run_workload, say, to_device
from linear_spatial_propagation_amd.inputs import (bf16_bits_to_f32, bf16_round_bits, make_workload)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_scan(x, w, lam, u, dtype, **kw):
    import torch
    import linear_spatial_propagation_amd as gspn
    t = [to_device(a, dtype) for a in (x, w, lam, u)]
    y = gspn.scan_fwd(*t, **kw)
    torch.cuda.synchronize()
    return from_device(y, dtype)


def store(a, dtype):
    a = np.asarray(a, dtype=np.float32)
    return bf16_round_bits(a) if dtype == "bf16" else a


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("H,W,g,path", [(64, 64, 1, 1), (32, 32, 1, 1), (56, 56, 1, 1), (64, 64, 4, 1),
                                        (128, 128, 8, 2), (37, 23, 1, 2), (64, 64, 1, 2)])
def test_ones_invariant(dtype, H, W, g, path):
    say(f"ones H={H} W={W} g={g} {dtype} path={path}")
    rng = np.random.default_rng(H + W + g)
    B, C = 2, 4
    one = np.ones((B, C, H, W), np.float32)
    w = 3 * rng.standard_normal((4, B, C, 3, H, W)).astype(np.float32)
    y = gpu_scan(store(one, dtype), store(w, dtype), store(one, dtype), store(one, dtype), dtype,
                 groups=g, path=path)
    expect = (H // g + 1) + (W // g + 1)
    if dtype == "bf16":
        assert np.all(y == expect), np.abs(y - expect).max()
    else:
        assert np.abs(y - expect).max() <= 1e-5 * expect


@pytest.mark.parametrize("path", [1, 2])
def test_groups_equal_lines_is_pointwise_exact(path):
    rng = np.random.default_rng(3)
    B, C, H, W = 2, 8, 32, 32
    x = rng.standard_normal((B, C, H, W)).astype(np.float32)
    lam, u = (rng.random((B, C, H, W)).astype(np.float32) for _ in range(2))
    w = rng.standard_normal((4, B, C, 3, H, W)).astype(np.float32)
    xs, ls, us, ws = (store(a, "bf16") for a in (x, lam, u, w))
    y = gpu_scan(xs, ws, ls, us, "bf16", groups=32, path=path)
    xf, lf, uf = (bf16_bits_to_f32(a).astype(np.float64) for a in (xs, ls, us))
    # u * 4 * lam * x is exact in fp32 for bf16 inputs, so the bf16 output is
    # exactly the round-to-nearest-even of the exact value
    expect = bf16_bits_to_f32(bf16_round_bits((uf * 4 * lf * xf).astype(np.float32))).astype(np.float64)
    np.testing.assert_array_equal(y, expect)


@pytest.mark.parametrize("path", [1, 2])
def test_hand_example(path):
    rows = {}
    with open(os.path.join(GOLDEN, "hand_2x3_tb.txt")) as f:
        for line in f:
            line = line.split("#")[0].split()
            if line:
                rows[line[0]] = [float(v) for v in line[1:]]
    H, W = int(rows["H"][0]), int(rows["W"][0])
    x = np.array(rows["x"], np.float32).reshape(1, 1, H, W)
    w = np.stack([np.array(rows[f"taps{t}"], np.float32).reshape(H, W) for t in range(3)])[None, None, None]
    one = np.ones_like(x)
    y = gpu_scan(x, np.ascontiguousarray(w), one, one, "f32", dirs=1, path=path)
    np.testing.assert_allclose(y.ravel(), rows["expect"], rtol=2e-6, atol=0)


@pytest.mark.parametrize("path", [1, 2])
def test_deterministic(path):
    wl = make_workload(4, 16, 64, 64, cpw=8, dtype="bf16", seed=21) if path == 1 else \
        make_workload(2, 4, 96, 96, dtype="bf16", seed=21)
    y1 = run_workload(wl, path)
    y2 = run_workload(wl, path)
    np.testing.assert_array_equal(y1, y2)


@pytest.mark.parametrize("path,H,W", [(1, 24, 40), (2, 24, 40), (2, 80, 70)])
def test_unused_taps_are_ignored(path, H, W):
    wl = make_workload(1, 2, H, W, dtype="f32", seed=4)
    y = run_workload(wl, path)
    w = wl.w_store.copy()
    nan, inf = np.float32("nan"), np.float32("inf")
    w[0:2, ..., 0, :, 0] = nan          # TB/BT tap 0 at column 0
    w[0:2, ..., 2, :, W - 1] = inf      # TB/BT tap 2 at column W-1
    w[2:4, ..., 0, 0, :] = -inf         # LR/RL tap 0 at row 0
    w[2:4, ..., 2, H - 1, :] = nan      # LR/RL tap 2 at row H-1
    w[0, ..., 0, :] = nan               # first lines of each direction
    w[1, ..., H - 1, :] = inf
    w[2, ..., :, 0] = -inf
    w[3, ..., :, W - 1] = nan
    wl.w_store = w
    np.testing.assert_array_equal(run_workload(wl, path), y)


@pytest.mark.parametrize("path", [1, 2])
def test_extreme_raw_taps(path):
    """Raw taps far outside N(0,1): the overflow-safe branches must agree
    with the exact definition."""
    rng = np.random.default_rng(6)
    B, C, H, W = 1, 3, 24, 24
    x = rng.standard_normal((B, C, H, W)).astype(np.float32)
    lam, u = (rng.random((B, C, H, W)).astype(np.float32) for _ in range(2))
    w = (rng.standard_normal((4, B, C, 3, H, W)) * 60).astype(np.float32)
    w[:, :, 1] -= 120.0     # whole rows of very negative taps
    y = gpu_scan(x, w, lam, u, "f32", path=path)
    yhat = oracle.scan_fwd(x, w, lam, u)
    assert parity_error(y, yhat, "f32") <= TOL["f32"]


def test_runs_on_a_side_stream():
    import torch
    import linear_spatial_propagation_amd as gspn
    wl = make_workload(2, 8, 64, 64, cpw=4, dtype="bf16", seed=8)
    t = [to_device(a, "bf16") for a in (wl.x_store, wl.w_store, wl.lam_store, wl.u_store)]
    ref = gspn.scan_fwd(*t, ch_per_weight=4)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        y = gspn.scan_fwd(*t, ch_per_weight=4)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)


def test_empty_like_inputs_rejected():
    import torch
    import linear_spatial_propagation_amd as gspn
    x = torch.zeros(1, 2, 0, 4, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(gspn.GspnError):
        gspn.scan_fwd(x, torch.zeros(4, 1, 2, 3, 0, 4, device="cuda", dtype=torch.bfloat16), x, x)
