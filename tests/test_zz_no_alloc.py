"""GPU test of gspn_scan_fwd_noalloc, the forward that allocates nothing.

Called through the C ABI (ctypes) on device buffers that torch allocates
beforehand.  Its output is compared with gspn_scan_fwd's on the same inputs
(the same kernels run, so bit for bit) and with the fp64 oracle at the parity
bound, on two calls in a row with the second on a smaller input (the static
scratch keeps the first call's contents).  A shape whose workspace exceeds
the scratch is rejected before any launch, with y untouched.
"""
import numpy as np
import pytest

import oracle
from parity import TOL, from_device, parity_error, say, to_device
from linear_spatial_propagation_amd import _lib
from linear_spatial_propagation_amd.inputs import make_workload

pytestmark = pytest.mark.gpu


def _run(wl, entry):
    import torch
    dt = _lib.GSPN_BF16 if wl.dtype == "bf16" else _lib.GSPN_F32
    x, w, lam, u = (to_device(a, wl.dtype) for a in (wl.x_store, wl.w_store, wl.lam_store, wl.u_store))
    y = torch.full_like(x, 7.0)
    stream = torch.cuda.current_stream().cuda_stream
    fn = _lib.scan_fwd_noalloc_ptr if entry == "noalloc" else _lib.scan_fwd_ptr
    rc = fn(x.data_ptr(), w.data_ptr(), lam.data_ptr(), u.data_ptr(), y.data_ptr(), wl.B, wl.C, wl.H, wl.W,
            dirs=wl.dirs, groups=wl.groups, ch_per_weight=wl.cpw, dtype=dt, stream=stream)
    torch.cuda.synchronize()
    return rc, from_device(y, wl.dtype)


SEQUENCES = [
    # two calls in a row on the line kernels, the second smaller
    [(2, 8, 128, 128, 15, 8, 1, "bf16"), (1, 3, 96, 64, 15, 1, 1, "bf16")],
    [(1, 4, 256, 200, 15, 1, 2, "f32"), (1, 2, 136, 72, 6, 2, 1, "f32")],
    # per-line fallback, then the fused path (no scratch), then the line kernels
    [(1, 2, 100, 37, 15, 1, 1, "bf16"), (2, 8, 64, 64, 15, 1, 4, "bf16"), (1, 1, 72, 80, 9, 1, 1, "bf16")],
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=lambda s: "_".join("x".join(map(str, c[:4])) for c in s))
def test_noalloc_matches_scan_fwd(seq):
    for i, (B, C, H, W, dirs, g, cpw, dtype) in enumerate(seq):
        say(f"noalloc call {i}: B={B} C={C} H={H} W={W} dirs={dirs} g={g} cpw={cpw} {dtype}")
        wl = make_workload(B, C, H, W, dirs=dirs, groups=g, cpw=cpw, dtype=dtype, seed=400 + i + B * C)
        rc, y = _run(wl, "noalloc")
        assert rc == 0, _lib.status_string(rc)
        rc2, y_ref = _run(wl, "plain")
        assert rc2 == 0
        np.testing.assert_array_equal(y, y_ref)
        yhat = oracle.scan_fwd(wl.x, wl.w, wl.lam, wl.u, dirs=dirs, groups=g, cpw=cpw)
        err = parity_error(y, yhat, dtype)
        say(f"  err {err:.3e}")
        assert err <= TOL[dtype]


def test_noalloc_rejects_a_workspace_beyond_the_scratch():
    import torch
    # 1 x 64 x 512 x 512 bf16 needs 4 * 64 * 512 * 512 * 4 bytes of planes alone
    B, C, H, W = 1, 64, 512, 512
    x = torch.zeros((B, C, H, W), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((4, B, C, 3, H, W), dtype=torch.bfloat16, device="cuda")
    y = torch.full_like(x, 3.0)
    rc = _lib.scan_fwd_noalloc_ptr(x.data_ptr(), w.data_ptr(), x.data_ptr(), x.data_ptr(), y.data_ptr(),
                                   B, C, H, W, dtype=_lib.GSPN_BF16)
    torch.cuda.synchronize()
    assert rc == _lib.ERR_SCRATCH
    assert "scratch" in _lib.load().gspn_last_error().decode()
    assert bool((y == 3.0).all())
