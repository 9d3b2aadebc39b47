"""GSPN 2D line-scan propagation on MI355X (gfx950).

    y = scan_fwd(x, w_raw, lam, u, dirs=15, groups=1, ch_per_weight=1)
    gx, gw_raw, glam, gu = scan_bwd(x, w_raw, lam, u, gy, dirs=15, groups=1, ch_per_weight=1)
    y = scan_fwd_dirs(x, w_raw, lam_d, u_d, ...)   # per-direction gains / gates
    ys = scan_fwd_batched([dict(x=..., w_raw=..., lam=..., u=...), ...])   # one launch
    y = gspn_scan(x, w_raw, lam, u, ...)   # differentiable: autograd runs scan_bwd
    z = block_fwd(x, w_in, w_out, ...)     # compressed block: projections around the scan

computes the 4-direction line recurrence of the Generalized Spatial
Propagation Network with hand-written HIP kernels (libgspn.so, C ABI in
include/gspn.h).  PyTorch supplies device memory and the current stream;
this wrapper only checks tensors and passes pointers.

Tensors (same dtype, float32 or bfloat16, contiguous, on one GPU):
  x, lam, u : [B, C, H, W]
  w_raw     : [popcount(dirs), B, C // ch_per_weight, 3, H, W]
"""
from __future__ import annotations

from . import _lib
from ._lib import (DIR_ALL, DIR_BT, DIR_LR, DIR_RL, DIR_TB, PATH_AUTO, PATH_FUSED, PATH_GENERAL, PATH_SLICE,
                   GspnError, load, select_path)

__all__ = ["scan_fwd", "scan_bwd", "scan_fwd_dirs", "scan_bwd_dirs", "scan_fwd_batched", "gspn_scan", "block_fwd",
           "block_rows", "select_path", "load", "GspnError", "DIR_TB", "DIR_BT", "DIR_LR", "DIR_RL",
           "DIR_ALL", "PATH_AUTO", "PATH_FUSED", "PATH_GENERAL", "PATH_SLICE"]


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return _lib.GSPN_BF16
    if t.dtype == torch.float32:
        return _lib.GSPN_F32
    raise TypeError(f"unsupported dtype {t.dtype}; use torch.bfloat16 or torch.float32")


def _check_inputs(tensors, dirs, ch_per_weight):
    x = tensors["x"]
    dev = x.device
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU (HIP) device")
    for name, t in tensors.items():
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, x is on {dev}")
        if t.dtype != x.dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, x has {x.dtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if x.dim() != 4:
        raise ValueError("x must be [B, C, H, W]")
    B, C, H, W = x.shape
    nd = bin(dirs & 15).count("1")
    for name, t in tensors.items():
        if name != "w_raw" and t.shape != x.shape:
            raise ValueError(f"{name} must have x's shape")
    if ch_per_weight < 1 or C % ch_per_weight:
        raise ValueError("ch_per_weight must divide C")
    w_raw = tensors["w_raw"]
    if tuple(w_raw.shape) != (nd, B, C // ch_per_weight, 3, H, W):
        raise ValueError(f"w_raw has shape {tuple(w_raw.shape)}, expected "
                         f"{(nd, B, C // ch_per_weight, 3, H, W)}")
    return dev, (B, C, H, W)


def scan_bwd(x, w_raw, lam, u, gy, *, dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1,
             out=None, path: int = PATH_AUTO):
    """Backward GSPN scan on the current HIP stream.

    Returns (gx, gw_raw, glam, gu), the gradients of a loss whose gradient
    with respect to y = scan_fwd(x, w_raw, lam, u) is gy.  ``out`` may give
    the four output tensors (contiguous, shaped like x, w_raw, x, x).
    """
    import torch
    dev, (B, C, H, W) = _check_inputs({"x": x, "w_raw": w_raw, "lam": lam, "u": u, "gy": gy},
                                      dirs, ch_per_weight)
    if out is None:
        gx, glam, gu = torch.empty_like(x), torch.empty_like(x), torch.empty_like(x)
        gw = torch.empty_like(w_raw)
    else:
        gx, gw, glam, gu = out
        for t, like in ((gx, x), (gw, w_raw), (glam, x), (gu, x)):
            if (t.shape != like.shape or t.dtype != like.dtype or t.device != dev
                    or not t.is_contiguous()):
                raise ValueError("out tensors must be contiguous and shaped like x, w_raw, x, x")
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = _lib.scan_bwd_ptr(x.data_ptr(), w_raw.data_ptr(), lam.data_ptr(), u.data_ptr(),
                               gy.data_ptr(), gx.data_ptr(), gw.data_ptr(), glam.data_ptr(),
                               gu.data_ptr(), B, C, H, W, dirs=dirs, groups=groups,
                               ch_per_weight=ch_per_weight, dtype=_dtype_code(x), path=path,
                               stream=stream)
    _lib.check(rc)
    return gx, gw, glam, gu


def scan_fwd_dirs(x, w_raw, lam, u, *, dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1,
                  out=None):
    """Forward scan with per-direction lambda and/or u (gspn_scan_fwd_ex).

    lam and u are each either [B, C, H, W] (shared by the directions) or
    [popcount(dirs), B, C, H, W] (one slab per enabled direction, ascending
    bit order); y = sum_d u_d * h_d with h_d driven by lam_d * x.
    """
    import torch
    if x.dim() != 4:
        raise ValueError("x must be [B, C, H, W]")
    nd = bin(dirs & 15).count("1")
    flags = 0
    shared = {"x": x, "w_raw": w_raw}
    for name, t, bit in (("lam", lam, _lib.LAM_PER_DIR), ("u", u, _lib.U_PER_DIR)):
        if t.dim() == 5:
            if tuple(t.shape) != (nd,) + tuple(x.shape):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(nd,) + tuple(x.shape)}")
            flags |= bit
            shared[name] = t[0]       # shape and dtype checks on one slab
        else:
            shared[name] = t
    dev, (B, C, H, W) = _check_inputs(shared, dirs, ch_per_weight)
    for name, t in (("lam", lam), ("u", u)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = _lib.scan_fwd_ex_ptr(x.data_ptr(), w_raw.data_ptr(), lam.data_ptr(), u.data_ptr(),
                                  out.data_ptr(), B, C, H, W, dirs=dirs, groups=groups,
                                  ch_per_weight=ch_per_weight, flags=flags, dtype=_dtype_code(x),
                                  stream=stream)
    _lib.check(rc)
    return out


def scan_bwd_dirs(x, w_raw, lam, u, gy, *, dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1,
                  out=None):
    """Backward of scan_fwd_dirs (gspn_scan_bwd_ex).

    lam and u as in scan_fwd_dirs; returns (gx, gw_raw, glam, gu) with glam
    and gu shaped like lam and u (one slab per enabled direction when that
    input has one).  ``out`` may give the four output tensors.
    """
    import torch
    if x.dim() != 4:
        raise ValueError("x must be [B, C, H, W]")
    nd = bin(dirs & 15).count("1")
    flags = 0
    shared = {"x": x, "w_raw": w_raw, "gy": gy}
    for name, t, bit in (("lam", lam, _lib.LAM_PER_DIR), ("u", u, _lib.U_PER_DIR)):
        if t.dim() == 5:
            if tuple(t.shape) != (nd,) + tuple(x.shape):
                raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {(nd,) + tuple(x.shape)}")
            flags |= bit
            shared[name] = t[0]       # shape and dtype checks on one slab
        else:
            shared[name] = t
    dev, (B, C, H, W) = _check_inputs(shared, dirs, ch_per_weight)
    for name, t in (("lam", lam), ("u", u)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if out is None:
        gx, gw, glam, gu = torch.empty_like(x), torch.empty_like(w_raw), torch.empty_like(lam), torch.empty_like(u)
    else:
        gx, gw, glam, gu = out
        for t, like in ((gx, x), (gw, w_raw), (glam, lam), (gu, u)):
            if (t.shape != like.shape or t.dtype != like.dtype or t.device != dev
                    or not t.is_contiguous()):
                raise ValueError("out tensors must be contiguous and shaped like x, w_raw, lam, u")
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = _lib.scan_bwd_ex_ptr(x.data_ptr(), w_raw.data_ptr(), lam.data_ptr(), u.data_ptr(),
                                  gy.data_ptr(), gx.data_ptr(), gw.data_ptr(), glam.data_ptr(),
                                  gu.data_ptr(), B, C, H, W, dirs=dirs, groups=groups,
                                  ch_per_weight=ch_per_weight, flags=flags, dtype=_dtype_code(x),
                                  stream=stream)
    _lib.check(rc)
    return gx, gw, glam, gu


def _autograd_function():
    import torch

    class _GspnScan(torch.autograd.Function):
        """y = scan_fwd(...) with scan_bwd as its backward (both HIP)."""

        @staticmethod
        def forward(ctx, x, w_raw, lam, u, dirs, groups, ch_per_weight):
            ctx.save_for_backward(x, w_raw, lam, u)
            ctx.opts = (dirs, groups, ch_per_weight)
            return scan_fwd(x, w_raw, lam, u, dirs=dirs, groups=groups, ch_per_weight=ch_per_weight)

        @staticmethod
        def backward(ctx, gy):
            x, w_raw, lam, u = ctx.saved_tensors
            dirs, groups, ch_per_weight = ctx.opts
            gx, gw, glam, gu = scan_bwd(x, w_raw, lam, u, gy.contiguous(), dirs=dirs, groups=groups,
                                        ch_per_weight=ch_per_weight)
            return gx, gw, glam, gu, None, None, None

    return _GspnScan


_GSPN_SCAN = None


def gspn_scan(x, w_raw, lam, u, *, dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1):
    """scan_fwd as a differentiable torch operation: autograd calls scan_bwd
    (the HIP backward) for the gradients of x, w_raw, lam and u."""
    global _GSPN_SCAN
    if _GSPN_SCAN is None:
        _GSPN_SCAN = _autograd_function()
    return _GSPN_SCAN.apply(x, w_raw, lam, u, dirs, groups, ch_per_weight)


def scan_fwd_batched(problems):
    """Several independent forward problems (each H, W <= 64) in one launch.

    problems: sequence of dicts with keys x, w_raw, lam, u and optionally
    dirs, groups, ch_per_weight, out.  All tensors share one dtype and
    device.  Returns the list of y tensors.
    """
    import torch
    if not problems:
        raise ValueError("no problems")
    structs, outs, dev, dt = [], [], None, None
    for pr in problems:
        dirs = pr.get("dirs", DIR_ALL)
        cpw = pr.get("ch_per_weight", 1)
        d, (B, C, H, W) = _check_inputs({"x": pr["x"], "w_raw": pr["w_raw"], "lam": pr["lam"], "u": pr["u"]},
                                        dirs, cpw)
        if dev is None:
            dev, dt = d, pr["x"].dtype
        elif d != dev or pr["x"].dtype != dt:
            raise ValueError("all problems must share one device and dtype")
        y = pr.get("out")
        if y is None:
            y = torch.empty_like(pr["x"])
        outs.append(y)
        structs.append(_lib.Problem(pr["x"].data_ptr(), pr["w_raw"].data_ptr(), pr["lam"].data_ptr(),
                                    pr["u"].data_ptr(), y.data_ptr(), B, C, H, W, dirs,
                                    pr.get("groups", 1), cpw))
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = _lib.scan_fwd_batched_ptr(structs, dtype=_dtype_code(problems[0]["x"]), stream=stream)
    _lib.check(rc)
    return outs


def scan_fwd(x, w_raw, lam, u, *, dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1,
             out=None, path: int = PATH_AUTO):
    """Forward GSPN scan on the current HIP stream; returns y [B, C, H, W]."""
    import torch
    dev, (B, C, H, W) = _check_inputs({"x": x, "w_raw": w_raw, "lam": lam, "u": u}, dirs, ch_per_weight)
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != dev or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    stream = torch.cuda.current_stream(dev).cuda_stream
    with torch.cuda.device(dev):
        rc = _lib.scan_fwd_ptr(x.data_ptr(), w_raw.data_ptr(), lam.data_ptr(), u.data_ptr(),
                               out.data_ptr(), B, C, H, W, dirs=dirs, groups=groups,
                               ch_per_weight=ch_per_weight, dtype=_dtype_code(x), path=path,
                               stream=stream)
    _lib.check(rc)
    return out


def block_rows(C_proxy: int, *, dirs: int = DIR_ALL, ch_per_weight: int = 1) -> int:
    """Rows of block_fwd's w_in: x_proxy, the raw taps of every enabled
    direction, lambda and u."""
    n = _lib.block_rows(C_proxy, dirs, ch_per_weight)
    _lib.check(n if n < 0 else 0)
    return n


def block_fwd(x, w_in, w_out, *, dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1,
              norm: bool = True, out=None):
    """The compressed propagation block (gspn_block_fwd) on the current stream.

    x: [B, C, H, W]; w_in: [block_rows(C_proxy), C]; w_out: [C, C_proxy];
    returns z: [B, C, H, W] = w_out (scan of the C_proxy-channel projection
    of x, with taps, lambda and u projected from x by the further rows of
    w_in), each pixel's scan output divided by its RMS over the C_proxy
    channels first when norm is set.
    """
    import torch
    for name, t in (("x", x), ("w_in", w_in), ("w_out", w_out)):
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU (HIP) device")
        if t.device != x.device or t.dtype != x.dtype:
            raise ValueError(f"{name} must share x's device and dtype")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if x.dim() != 4 or w_in.dim() != 2 or w_out.dim() != 2:
        raise ValueError("x must be [B, C, H, W], w_in and w_out matrices")
    B, C, H, W = x.shape
    Cp = w_out.shape[1]
    rows = block_rows(Cp, dirs=dirs, ch_per_weight=ch_per_weight)
    if tuple(w_out.shape) != (C, Cp) or tuple(w_in.shape) != (rows, C):
        raise ValueError(f"w_in must be [{rows}, {C}] and w_out [{C}, {Cp}]")
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or out.device != x.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like x")
    stream = torch.cuda.current_stream(x.device).cuda_stream
    with torch.cuda.device(x.device):
        rc = _lib.block_fwd_ptr(x.data_ptr(), w_in.data_ptr(), w_out.data_ptr(), out.data_ptr(), B, C, Cp, H, W,
                                dirs=dirs, groups=groups, ch_per_weight=ch_per_weight,
                                flags=_lib.BLOCK_RMSNORM if norm else 0, dtype=_dtype_code(x), stream=stream)
    _lib.check(rc)
    return out
