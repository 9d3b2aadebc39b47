"""Pins of the oracle's one-slice entry point and of the one-slice input
generator, no GPU.

The two largest workloads (2K local groups, 512 x 512 generation scale) are
checked on the GPU slice by slice: the oracle recomputes single (b, c)
slices with ``oracle.slice_fwd`` from inputs regenerated alone by
``inputs.slice_inputs_f64``.  Both are tied here, bit for bit, to the
whole-tensor path that the dense closed form and the invariants pin
(``oracle.scan_fwd`` on ``make_workload``): the slice path adds no
arithmetic of its own, and regenerating one slice reproduces exactly the
values the whole tensor holds at that slice.
"""
import numpy as np
import pytest

import oracle
from linear_spatial_propagation_amd.inputs import enabled_dirs, make_workload, slice_inputs_f64

CASES = [
    # B, C, H, W, dirs, groups, cpw, dtype, u_ones
    (2, 4, 12, 10, 15, 1, 1, "bf16", False),
    (2, 4, 12, 10, 15, 1, 1, "f32", False),
    (1, 6, 16, 8, 15, 4, 3, "bf16", False),     # local groups, shared weights
    (2, 4, 8, 16, 15, 2, 2, "f32", True),       # u = 1
    (1, 4, 9, 7, 5, 1, 2, "bf16", False),       # TB + LR
    (1, 3, 10, 6, 10, 2, 1, "f32", False),      # BT + RL
    (2, 2, 6, 12, 8, 3, 1, "bf16", True),       # RL alone, three groups
    (1, 8, 8, 8, 15, 8, 8, "bf16", False),      # g = n, one set for all channels
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(map(str, c)))
def test_slice_path_equals_whole_tensor(case):
    B, C, H, W, dirs, groups, cpw, dtype, u_ones = case
    seed = 31 + sum(int(v) for v in case[:7])
    wl = make_workload(B, C, H, W, dirs=dirs, groups=groups, cpw=cpw, dtype=dtype, seed=seed,
                       u_ones=u_ones)
    y = oracle.scan_fwd(wl.x, wl.w, wl.lam, wl.u, dirs=dirs, groups=groups, cpw=cpw)
    nd = len(enabled_dirs(dirs))
    for b in range(B):
        for c in range(C):
            x, w, lam, u = slice_inputs_f64(seed, b, c, H=H, W=W, dirs=dirs, cpw=cpw, dtype=dtype,
                                            u_ones=u_ones)
            # the regenerated slice is the whole tensor's slice, bit for bit
            np.testing.assert_array_equal(x, wl.x[b, c])
            np.testing.assert_array_equal(lam, wl.lam[b, c])
            np.testing.assert_array_equal(u, wl.u[b, c])
            assert w.shape == (nd, 3, H, W)
            np.testing.assert_array_equal(w, wl.w[:, b, c // cpw])
            # and the one-slice oracle is the whole-tensor oracle at that slice
            np.testing.assert_array_equal(oracle.slice_fwd(x, w, lam, u, dirs=dirs, groups=groups), y[b, c])


def test_slice_generator_distinguishes_slices_and_sets():
    # a wrong index in the per-slice streams (b and c swapped, or the weight
    # set taken as c instead of c // cpw) must change the regenerated values
    kw = dict(H=6, W=6, dirs=15, cpw=2, dtype="f32")
    x01, w01, _, _ = slice_inputs_f64(3, 0, 1, **kw)
    x10, _, _, _ = slice_inputs_f64(3, 1, 0, **kw)
    assert not np.array_equal(x01, x10)
    _, w00, _, _ = slice_inputs_f64(3, 0, 0, **kw)
    _, w02, _, _ = slice_inputs_f64(3, 0, 2, **kw)
    np.testing.assert_array_equal(w00, w01)     # channels 0 and 1 share set 0
    assert not np.array_equal(w01, w02)         # channel 2 uses set 1
