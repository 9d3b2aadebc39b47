"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects every invalid argument on the host before any launch.

Calls here only pass invalid arguments (or fake pointers with invalid
arguments), which the library rejects before touching the HIP runtime.
"""
import ctypes
import os
import re

import pytest

import linear_spatial_propagation_amd as gspn
from linear_spatial_propagation_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gspn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gspn_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from linear_spatial_propagation_amd import build
        build.build()
    return _lib.load()


def test_header_declares_expected_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_version_and_strings(lib):
    assert lib.gspn_version() == 1
    for code in range(0, -13, -1):
        s = _lib.status_string(code)
        assert s.startswith("GSPN_"), (code, s)
    assert "unknown" in _lib.status_string(-99)


FAKE = 1 << 40  # 16-byte aligned, never dereferenced: every call below fails validation first


def call(**kw):
    args = dict(x=FAKE, w=FAKE + (1 << 32), lam=FAKE + (2 << 32), u=FAKE + (3 << 32), y=FAKE + (4 << 32),
                B=2, C=8, H=16, W=16, dirs=15, groups=1, ch_per_weight=1, dtype=1, path=0)
    args.update(kw)
    return _lib.scan_fwd_ptr(args["x"], args["w"], args["lam"], args["u"], args["y"], args["B"],
                             args["C"], args["H"], args["W"], dirs=args["dirs"], groups=args["groups"],
                             ch_per_weight=args["ch_per_weight"], dtype=args["dtype"], path=args["path"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(C=-1), -2), (dict(H=0), -2), (dict(W=4097), -2), (dict(H=5000), -2),
    (dict(B=1 << 20, C=1 << 20), -2),
    (dict(dirs=0), -3), (dict(dirs=16), -3), (dict(dirs=0x1F), -3),
    (dict(groups=0), -4), (dict(groups=3), -4), (dict(H=12, groups=8, dirs=1), -4),
    (dict(W=12, groups=8, dirs=4), -4),
    (dict(ch_per_weight=0), -5), (dict(ch_per_weight=3), -5),
    (dict(dtype=2), -6), (dict(dtype=-1), -6),
    (dict(x=0), -1), (dict(w=0), -1), (dict(y=0), -1), (dict(lam=0), -1), (dict(u=0), -1),
    (dict(x=FAKE + 8), -7), (dict(y=FAKE + (4 << 32) + 2), -7),
    (dict(y=FAKE), -8), (dict(y=FAKE + (3 << 32) + 64), -8),
    (dict(path=7), -10), (dict(path=1, H=65), -10),
])
def test_invalid_arguments_rejected_on_host(lib, kw, code):
    assert call(**kw) == code


def test_groups_only_checked_on_scanned_sides(lib):
    # H=12 is not divisible by 8, but only LR/RL scan W=16: the size check
    # passes, so the call proceeds to the pointer checks (aliasing here)
    assert call(H=12, W=16, groups=8, dirs=12, y=FAKE) == -8


def test_select_path(lib):
    assert gspn.select_path(32, 128, 64, 64, ch_per_weight=8) == gspn.PATH_FUSED
    assert gspn.select_path(1, 8, 32, 32) == gspn.PATH_FUSED
    assert gspn.select_path(8, 256, 128, 128, groups=8) == gspn.PATH_SLICE
    assert gspn.select_path(8, 256, 128, 128, groups=8, dtype=0) == gspn.PATH_GENERAL   # fp32
    assert gspn.select_path(8, 256, 128, 128, groups=4) == gspn.PATH_GENERAL            # too few groups
    assert gspn.select_path(1, 320, 512, 512) == gspn.PATH_GENERAL
    assert gspn.select_path(1, 8, 32, 32, dirs=0) == -3


def test_python_wrapper_rejects_bad_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 4, 4)
    with pytest.raises(ValueError):
        gspn.scan_fwd(x, torch.zeros(4, 1, 2, 3, 4, 4), x, x)  # CPU tensors


def test_check_raises_with_status(lib):
    with pytest.raises(gspn.GspnError) as ei:
        _lib.check(-4)
    assert ei.value.status == -4


def call_bwd(**kw):
    names = ("x", "w", "lam", "u", "gy", "gx", "gw", "glam", "gu")
    args = {nm: FAKE + (i << 32) for i, nm in enumerate(names)}
    args.update(B=2, C=8, H=16, W=16, dirs=15, groups=1, ch_per_weight=1, dtype=1, path=0)
    args.update(kw)
    return _lib.scan_bwd_ptr(*(args[nm] for nm in names), args["B"], args["C"], args["H"], args["W"],
                             dirs=args["dirs"], groups=args["groups"],
                             ch_per_weight=args["ch_per_weight"], dtype=args["dtype"], path=args["path"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(W=4097), -2), (dict(dirs=0), -3), (dict(groups=3), -4),
    (dict(ch_per_weight=3), -5), (dict(dtype=2), -6),
    (dict(x=0), -1), (dict(gy=0), -1), (dict(gx=0), -1), (dict(gw=0), -1), (dict(glam=0), -1),
    (dict(gu=0), -1),
    (dict(gy=FAKE + 8), -7), (dict(gw=FAKE + (6 << 32) + 4), -7),
    (dict(gx=FAKE), -8),                          # output on an input
    (dict(gu=FAKE + (4 << 32) + 512), -8),        # output inside gy
    (dict(glam=FAKE + (5 << 32) + 16), -8),       # two outputs overlap
    (dict(gw=FAKE + (1 << 32)), -8),              # tap gradients on the taps
    (dict(H=1000, W=16), -10), (dict(H=130, W=16), -10), (dict(H=600, W=600), -10),
    (dict(path=7), -10), (dict(path=1, W=65), -10), (dict(path=2, H=130), -10),
])
def test_bwd_invalid_arguments_rejected_on_host(lib, kw, code):
    assert call_bwd(**kw) == code


def test_bwd_supported(lib):
    assert _lib.bwd_supported(32, 128, 64, 64, ch_per_weight=8) == 0
    assert _lib.bwd_supported(64, 96, 56, 56) == 0
    assert _lib.bwd_supported(8, 256, 128, 128, groups=8) == 0
    assert _lib.bwd_supported(1, 320, 512, 512) == 0
    assert _lib.bwd_supported(1, 8, 130, 64) == -10     # 130 is not a multiple of K = 4
    assert _lib.bwd_supported(1, 8, 513, 64) == -10
    assert _lib.bwd_supported(1, 8, 32, 32, groups=5) == -4


def call_ex(**kw):
    args = dict(x=FAKE, w=FAKE + (1 << 32), lam=FAKE + (2 << 32), u=FAKE + (3 << 32), y=FAKE + (4 << 32),
                B=2, C=8, H=16, W=16, dirs=15, groups=1, ch_per_weight=1, flags=1, dtype=1)
    args.update(kw)
    return _lib.scan_fwd_ex_ptr(args["x"], args["w"], args["lam"], args["u"], args["y"], args["B"],
                                args["C"], args["H"], args["W"], dirs=args["dirs"], groups=args["groups"],
                                ch_per_weight=args["ch_per_weight"], flags=args["flags"],
                                dtype=args["dtype"])


NBYTES = 2 * 8 * 16 * 16 * 2   # one bf16 [B][C][H][W] slab of call_ex's default shape


@pytest.mark.parametrize("kw,code", [
    (dict(flags=4), -11), (dict(flags=0xFF), -11),
    (dict(B=0), -2), (dict(dirs=0), -3), (dict(groups=3), -4), (dict(ch_per_weight=3), -5),
    (dict(dtype=2), -6), (dict(lam=0), -1), (dict(u=0), -1), (dict(x=FAKE + 4), -7),
    (dict(y=FAKE + (2 << 32) + NBYTES), -8),             # y inside the second lambda slab
    (dict(flags=2, y=FAKE + (3 << 32) + 3 * NBYTES), -8), # y inside the last gate slab
    (dict(H=130), -10), (dict(flags=3, W=600), -10),
])
def test_variant_invalid_arguments_rejected_on_host(lib, kw, code):
    assert call_ex(**kw) == code


def test_python_variant_wrapper_rejects_bad_shapes():
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 2, 4, 4)
    with pytest.raises(ValueError):
        gspn.scan_fwd_dirs(x, torch.zeros(4, 1, 2, 3, 4, 4), torch.zeros(3, 1, 2, 4, 4), x)


def prob(i=0, **kw):
    base = FAKE + (i << 36)
    d = dict(x=base, w_raw=base + (1 << 32), lam=base + (2 << 32), u=base + (3 << 32), y=base + (4 << 32),
             B=2, C=8, H=16, W=16, dirs=15, groups=1, ch_per_weight=1)
    d.update(kw)
    return _lib.Problem(**d)


@pytest.mark.parametrize("probs,kw,code", [
    ([], {}, -2),
    ([prob(i) for i in range(33)], {}, -2),
    ([prob(0)], dict(dtype=3), -6),
    ([prob(0), prob(1, H=65)], {}, -10),
    ([prob(0), prob(1, groups=3)], {}, -4),
    ([prob(0), prob(1, x=0)], {}, -1),
    ([prob(0), prob(1, y=FAKE + (1 << 36) + (4 << 32) + 8)], {}, -7),
    ([prob(0), prob(1, y=FAKE + (2 << 32))], {}, -8),              # y of problem 1 on lam of problem 0
    ([prob(0), prob(1, y=FAKE + (4 << 32) + 256)], {}, -8),        # the two outputs overlap
])
def test_batched_invalid_arguments_rejected_on_host(lib, probs, kw, code):
    assert _lib.scan_fwd_batched_ptr(probs, **kw) == code


def call_bwd_ex(**kw):
    names = ("x", "w", "lam", "u", "gy", "gx", "gw", "glam", "gu")
    args = {nm: FAKE + (i << 32) for i, nm in enumerate(names)}
    args.update(B=2, C=8, H=16, W=16, dirs=15, groups=1, ch_per_weight=1, flags=3, dtype=1)
    args.update(kw)
    return _lib.scan_bwd_ex_ptr(*(args[nm] for nm in names), args["B"], args["C"], args["H"], args["W"],
                                dirs=args["dirs"], groups=args["groups"], ch_per_weight=args["ch_per_weight"],
                                flags=args["flags"], dtype=args["dtype"])


@pytest.mark.parametrize("kw,code", [
    (dict(flags=4), -11), (dict(flags=0x10), -11),
    (dict(B=0), -2), (dict(dirs=0), -3), (dict(groups=3), -4), (dict(ch_per_weight=3), -5),
    (dict(dtype=2), -6), (dict(lam=0), -1), (dict(gu=0), -1), (dict(glam=FAKE + (7 << 32) + 4), -7),
    (dict(gx=FAKE + (2 << 32) + 3 * NBYTES), -8),           # gx inside the last lambda slab
    (dict(gx=FAKE + (8 << 32) + 2 * NBYTES), -8),           # gx inside the third gu slab
    (dict(H=130), -10), (dict(flags=3, W=600), -10),
])
def test_variant_bwd_invalid_arguments_rejected_on_host(lib, kw, code):
    assert call_bwd_ex(**kw) == code


def test_variant_bwd_flags_zero_is_the_shared_backward(lib):
    assert call_bwd_ex(flags=0, H=130) == call_bwd(H=130) == -10
    assert call_bwd_ex(flags=0, gx=FAKE) == -8


def call_block(**kw):
    args = dict(x=FAKE, w_in=FAKE + (1 << 32), w_out=FAKE + (2 << 32), z=FAKE + (3 << 32), B=2, C=24, C_proxy=8,
                H=16, W=16, dirs=15, groups=1, ch_per_weight=2, flags=1, dtype=1)
    args.update(kw)
    return _lib.block_fwd_ptr(args["x"], args["w_in"], args["w_out"], args["z"], args["B"], args["C"],
                              args["C_proxy"], args["H"], args["W"], dirs=args["dirs"], groups=args["groups"],
                              ch_per_weight=args["ch_per_weight"], flags=args["flags"], dtype=args["dtype"])


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), -2), (dict(C=0), -2), (dict(C_proxy=0), -2), (dict(W=4097), -2), (dict(B=1 << 20, C=1 << 10), -2),
    (dict(dirs=0), -3), (dict(dirs=16), -3), (dict(groups=3), -4), (dict(ch_per_weight=3), -5),
    (dict(dtype=2), -6), (dict(x=0), -1), (dict(w_in=0), -1), (dict(w_out=0), -1), (dict(z=0), -1),
    (dict(z=FAKE + (3 << 32) + 8), -7), (dict(flags=2), -11), (dict(flags=0x80000001), -11),
    (dict(z=FAKE), -8),                              # z on x
    (dict(z=FAKE + (1 << 32) + 1024), -8),           # z inside w_in
    (dict(z=FAKE + (2 << 32) - 256), -8),            # z runs into w_out
])
def test_block_invalid_arguments_rejected_on_host(lib, kw, code):
    assert call_block(**kw) == code


def test_block_rows(lib):
    assert _lib.block_rows(128, 15, 8) == 3 * 128 + 3 * 4 * 16
    assert _lib.block_rows(8, 5, 2) == 24 + 3 * 2 * 4
    assert _lib.block_rows(0, 15, 1) == -2
    assert _lib.block_rows(8, 0, 1) == -3
    assert _lib.block_rows(8, 15, 3) == -5
