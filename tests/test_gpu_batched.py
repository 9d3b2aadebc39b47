"""GPU tests of the batched forward (gspn_scan_fwd_batched): several small
problems in one launch give the same results as separate gspn_scan_fwd
calls (the same kernel code runs every problem), and match the oracle."""
import numpy as np
import pytest

import oracle
from parity import TOL, from_device, parity_error, say, to_device
from linear_spatial_propagation_amd.inputs import make_workload

pytestmark = pytest.mark.gpu


def problems_of(shapes, dtype):
    wls = [make_workload(B, C, H, W, dirs=d, groups=g, cpw=cpw, dtype=dtype, seed=100 + i)
           for i, (B, C, H, W, d, g, cpw) in enumerate(shapes)]
    probs = []
    for wl in wls:
        probs.append(dict(x=to_device(wl.x_store, dtype), w_raw=to_device(wl.w_store, dtype),
                          lam=to_device(wl.lam_store, dtype), u=to_device(wl.u_store, dtype),
                          dirs=wl.dirs, groups=wl.groups, ch_per_weight=wl.cpw))
    return wls, probs


MIXES = {
    "tiny16": [(1, 8, 32, 32, 15, 1, 1)] * 16,
    "mixed": [(1, 8, 32, 32, 15, 1, 1), (2, 16, 64, 64, 15, 1, 8), (1, 4, 20, 30, 5, 2, 2),
              (1, 3, 17, 45, 15, 1, 3), (2, 2, 64, 64, 15, 64, 1), (1, 2, 1, 7, 15, 1, 1)],
    "vec_rows": [(1, 8, 32, 32, 15, 1, 1), (1, 4, 56, 56, 12, 1, 2), (2, 8, 64, 48, 3, 4, 4)],
}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("mix", sorted(MIXES))
def test_batched_equals_separate_calls_and_oracle(mix, dtype):
    import torch
    import linear_spatial_propagation_amd as gspn
    say(f"case batched {mix} {dtype}")
    wls, probs = problems_of(MIXES[mix], dtype)
    ys = gspn.scan_fwd_batched(probs)
    singles = [gspn.scan_fwd(p["x"], p["w_raw"], p["lam"], p["u"], dirs=p["dirs"], groups=p["groups"],
                             ch_per_weight=p["ch_per_weight"]) for p in probs]
    torch.cuda.synchronize()
    for wl, y, y1 in zip(wls, ys, singles):
        a, b = from_device(y, dtype), from_device(y1, dtype)
        if MIXES[mix] and all(s[3] % (8 if dtype == "bf16" else 4) == 0 for s in MIXES[mix]):
            # the same kernel instantiation ran both: bit-identical
            np.testing.assert_array_equal(a, b)
        yhat = oracle.scan_fwd(wl.x, wl.w, wl.lam, wl.u, dirs=wl.dirs, groups=wl.groups, cpw=wl.cpw)
        err = parity_error(a, yhat, dtype)
        assert err <= TOL[dtype], err


def test_batched_maximum_count():
    import torch
    import linear_spatial_propagation_amd as gspn
    wls, probs = problems_of([(1, 2, 16, 24, 15, 1, 1)] * 32, "f32")
    ys = gspn.scan_fwd_batched(probs)
    torch.cuda.synchronize()
    for wl, y in zip(wls, ys):
        yhat = oracle.scan_fwd(wl.x, wl.w, wl.lam, wl.u)
        assert parity_error(from_device(y, "f32"), yhat, "f32") <= TOL["f32"]
