"""fp64 CPU oracle for the GSPN 4-direction line scan -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package.  The HIP library never imports, links or calls it.

The arithmetic lives in ``gspn_oracle.c`` (plain C loops in fp64, OpenMP over
(b, c) slices); this module compiles it with gcc and calls it through ctypes.
Its header lists the passages of the pages it follows and the readings taken
where they are silent.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gspn_oracle.c")
_LIB = os.path.join(_HERE, "libgspn_oracle.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle library in place (gcc, -O2, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def open_library(path: str):
    """ctypes handle of an oracle library built from ``gspn_oracle.c``."""
    lib = ctypes.CDLL(path)
    dp = ctypes.POINTER(ctypes.c_double)
    lib.gspn_oracle_fwd_f64.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_int64, ctypes.c_uint32,
                                        ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
    lib.gspn_oracle_fwd_f64.restype = ctypes.c_int
    lib.gspn_oracle_slice_f64.argtypes = [dp, dp, dp, dp, dp, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_uint32, ctypes.c_int32]
    lib.gspn_oracle_slice_f64.restype = ctypes.c_int
    lib.gspn_oracle_bwd_f64.argtypes = [dp] * 9 + [ctypes.c_int64] * 4 + [
        ctypes.c_uint32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int]
    lib.gspn_oracle_bwd_f64.restype = ctypes.c_int
    lib.gspn_oracle_max_threads.argtypes = []
    lib.gspn_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    with _lock:
        if _lib is None:
            build()
            _lib = open_library(_LIB)
    return _lib


def _dptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64c(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def max_threads() -> int:
    return _load().gspn_oracle_max_threads()


def scan_fwd(x, w, lam, u, *, dirs: int = 15, groups: int = 1, cpw: int = 1,
             nthreads: int = 0, lib=None) -> np.ndarray:
    """y[B][C][H][W] in fp64.

    x, lam, u: [B][C][H][W]; w: [popcount(dirs)][B][C/cpw][3][H][W].
    """
    x, w, lam, u = (_f64c(a) for a in (x, w, lam, u))
    B, C, H, W = x.shape
    nd = bin(dirs & 15).count("1")
    if lam.shape != x.shape or u.shape != x.shape:
        raise ValueError("x, lam, u must share one shape")
    if cpw < 1 or C % cpw or w.shape != (nd, B, C // cpw, 3, H, W):
        raise ValueError(f"w has shape {w.shape}, expected {(nd, B, C // max(cpw, 1), 3, H, W)}")
    y = np.empty_like(x)
    rc = (lib or _load()).gspn_oracle_fwd_f64(_dptr(x), _dptr(w), _dptr(lam), _dptr(u), _dptr(y),
                                     B, C, H, W, dirs, groups, cpw, nthreads)
    if rc:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return y


def scan_fwd_dirs(x, w, lam, u, *, dirs: int = 15, groups: int = 1, cpw: int = 1,
                  nthreads: int = 0) -> np.ndarray:
    """Per-direction variant: y = sum_d u_d * h_d, h_d driven by lam_d * x.

    lam and u are [B][C][H][W] (shared) or [popcount(dirs)][B][C][H][W].
    Written as the sum of single-direction calls of the oracle above, which
    computes u_d * h_d for one direction exactly as the definition states.
    """
    x, w, lam, u = (_f64c(a) for a in (x, w, lam, u))
    y = np.zeros_like(x)
    slab = 0
    for d in range(4):
        if not (dirs >> d) & 1:
            continue
        lam_d = lam[slab] if lam.ndim == 5 else lam
        u_d = u[slab] if u.ndim == 5 else u
        y += scan_fwd(x, w[slab:slab + 1], lam_d, u_d, dirs=1 << d, groups=groups, cpw=cpw,
                      nthreads=nthreads)
        slab += 1
    return y


def scan_bwd(x, w, lam, u, gy, *, dirs: int = 15, groups: int = 1, cpw: int = 1,
             nthreads: int = 0, lib=None):
    """Gradients (gx, gw, glam, gu) in fp64 of L with dL/dy = gy.

    Shapes as in scan_fwd; gw is dL/d(raw taps), shaped like w, with zeros on
    the taps the forward never reads.
    """
    x, w, lam, u, gy = (_f64c(a) for a in (x, w, lam, u, gy))
    B, C, H, W = x.shape
    nd = bin(dirs & 15).count("1")
    if lam.shape != x.shape or u.shape != x.shape or gy.shape != x.shape:
        raise ValueError("x, lam, u, gy must share one shape")
    if cpw < 1 or C % cpw or w.shape != (nd, B, C // cpw, 3, H, W):
        raise ValueError(f"w has shape {w.shape}, expected {(nd, B, C // max(cpw, 1), 3, H, W)}")
    gx, glam, gu = np.empty_like(x), np.empty_like(x), np.empty_like(x)
    gw = np.empty_like(w)
    rc = (lib or _load()).gspn_oracle_bwd_f64(
        _dptr(x), _dptr(w), _dptr(lam), _dptr(u), _dptr(gy), _dptr(gx), _dptr(gw), _dptr(glam),
        _dptr(gu), B, C, H, W, dirs, groups, cpw, nthreads)
    if rc:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return gx, gw, glam, gu


def scan_bwd_dirs(x, w, lam, u, gy, *, dirs: int = 15, groups: int = 1, cpw: int = 1,
                  nthreads: int = 0, lib=None):
    """Gradients (gx, gw, glam, gu) in fp64 of the per-direction variant
    y = sum_d u_d * h_d, h_d driven by lam_d * x, for dL/dy = gy.

    lam and u are [B][C][H][W] (shared) or [popcount(dirs)][B][C][H][W];
    glam and gu have the shapes of lam and u.  y is the sum of
    single-direction scans, each reading x, its own slab of w, lam_d and u_d,
    so each gradient is the sum over directions of the single-direction
    backward above (a shared lam or u collects every direction's term).
    """
    x, w, lam, u, gy = (_f64c(a) for a in (x, w, lam, u, gy))
    gx = np.zeros_like(x)
    gw = np.empty_like(w)
    glam = np.zeros_like(lam)
    gu = np.zeros_like(u)
    slab = 0
    for d in range(4):
        if not (dirs >> d) & 1:
            continue
        lam_d = lam[slab] if lam.ndim == 5 else lam
        u_d = u[slab] if u.ndim == 5 else u
        gx_d, gw_d, glam_d, gu_d = scan_bwd(x, w[slab:slab + 1], lam_d, u_d, gy, dirs=1 << d, groups=groups,
                                            cpw=cpw, nthreads=nthreads, lib=lib)
        gx += gx_d
        gw[slab] = gw_d[0]
        if lam.ndim == 5:
            glam[slab] = glam_d
        else:
            glam += glam_d
        if u.ndim == 5:
            gu[slab] = gu_d
        else:
            gu += gu_d
        slab += 1
    return gx, gw, glam, gu



def round_bf16(a) -> np.ndarray:
    """Values rounded to bfloat16 (round to nearest, ties to even), in fp64.

    The fp64 value is first rounded to fp32 (numpy's conversion rounds to
    nearest even), then its low 16 bits are rounded away, ties to even.
    """
    f = np.ascontiguousarray(a, dtype=np.float32)
    b = f.view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000
    return b.astype(np.uint32).view(np.float32).astype(np.float64)


def block_rows(C_proxy: int, dirs: int, cpw: int) -> int:
    """Rows of the block's input projection: proxy, taps, lambda, u."""
    nd = bin(dirs & 15).count("1")
    return C_proxy + nd * (C_proxy // cpw) * 3 + 2 * C_proxy


BLOCK_NORM_EPS = 1e-6


def block_fwd(x, w_in, w_out, *, dirs: int = 15, groups: int = 1, cpw: int = 1, norm: bool = True,
              io_round=None, nthreads: int = 0, lib=None) -> np.ndarray:
    """The compressed propagation block around the scan, in fp64.

    Reading of the block (GSPN-2 response, *Relate Compressive Proxy
    Dimension to Low-rank Approximation*; C-GSPN abstract): per pixel, one
    linear layer maps the C input channels to x_proxy (C_proxy channels),
    the raw taps, lambda and u; the scan runs over x_proxy; a second linear
    layer maps its C_proxy output channels back to C.  With norm (the
    block's "fused normalization", C-GSPN abstract, read as an RMS
    normalisation in the compressed space): before the output projection the
    scan output of each pixel is divided by its root mean square over the
    C_proxy channels, sqrt(mean_c y_c^2 + BLOCK_NORM_EPS); no learned gain
    (a per-channel gain is a diagonal factor that w_out absorbs).

    x: [B][C][H][W]; w_in: [block_rows][C], rows in the order x_proxy
    (C_proxy), the raw taps (one slab per enabled direction, TB, BT, LR, RL;
    within a slab set k and tap t at row k*3 + t), lambda (C_proxy), u
    (C_proxy); w_out: [C][C_proxy].  Returns z: [B][C][H][W].

    io_round: None for exact fp64 throughout, or a function applied to the
    four generated tensors and to the scan output, the rounding of a block
    that stores them in a narrower dtype (round_bf16 for bf16 storage).
    """
    x, w_in, w_out = (_f64c(a) for a in (x, w_in, w_out))
    B, C, H, W = x.shape
    Cp = w_out.shape[1]
    nd = bin(dirs & 15).count("1")
    if w_out.shape != (C, Cp) or cpw < 1 or Cp % cpw:
        raise ValueError(f"w_out has shape {w_out.shape}; C_proxy must be a multiple of cpw")
    Cw = Cp // cpw
    if w_in.shape != (block_rows(Cp, dirs, cpw), C):
        raise ValueError(f"w_in has shape {w_in.shape}, expected {(block_rows(Cp, dirs, cpw), C)}")
    rnd = io_round or (lambda a: a)
    g = np.matmul(w_in, x.reshape(B, C, H * W))            # [B][rows][HW]
    t0, t1 = Cp, Cp + nd * Cw * 3
    xp = rnd(g[:, :Cp]).reshape(B, Cp, H, W)
    taps = rnd(g[:, t0:t1]).reshape(B, nd, Cw, 3, H, W).transpose(1, 0, 2, 3, 4, 5)
    lam = rnd(g[:, t1:t1 + Cp]).reshape(B, Cp, H, W)
    u = rnd(g[:, t1 + Cp:]).reshape(B, Cp, H, W)
    y = rnd(scan_fwd(xp, taps, lam, u, dirs=dirs, groups=groups, cpw=cpw, nthreads=nthreads, lib=lib))
    y = y.reshape(B, Cp, H * W)
    if norm:
        y = y / np.sqrt(np.mean(y * y, axis=1, keepdims=True) + BLOCK_NORM_EPS)
    return np.matmul(w_out, y).reshape(B, C, H, W)

def slice_fwd(x, w, lam, u, *, dirs: int = 15, groups: int = 1) -> np.ndarray:
    """One slice: x, lam, u [H][W]; w [popcount(dirs)][3][H][W] -> y [H][W]."""
    x, w, lam, u = (_f64c(a) for a in (x, w, lam, u))
    H, W = x.shape
    nd = bin(dirs & 15).count("1")
    if w.shape != (nd, 3, H, W):
        raise ValueError(f"w has shape {w.shape}, expected {(nd, 3, H, W)}")
    y = np.empty_like(x)
    rc = _load().gspn_oracle_slice_f64(_dptr(x), _dptr(w), _dptr(lam), _dptr(u), _dptr(y),
                                       H, W, dirs, groups)
    if rc:
        raise ValueError(f"oracle rejected the arguments (code {rc})")
    return y
