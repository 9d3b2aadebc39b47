"""Seeded synthetic inputs for the GSPN line-scan operator.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the operator's arithmetic, so both the fp64 oracle (tests)
and the HIP path (tests, benchmark) can consume the same tensors.

Layouts (all C-contiguous):
  x, lam, u : [B][C][H][W]
  w_raw     : [ndir][B][C/cpw][3][H][W], one slab per enabled direction in
              ascending bit order (TB=1, BT=2, LR=4, RL=8).

Streams are per slice so that any slice can be regenerated alone:
  x, lam, u of slice (b, c)      <- default_rng([seed, 0, b, c]), drawn in
                                    the order x, lam, u;
  w_raw of (direction bit d, b, k) <- default_rng([seed, 1, d, b, k]).
  the upstream gradient gy of slice (b, c) <- default_rng([seed, 2, b, c]).
Value distributions: x ~ N(0, 1), raw taps ~ N(0, 1), lam ~ U(0, 1),
u ~ U(0, 1) (or u = 1), gy ~ N(0, 1).  Values are drawn in float32 and, for bf16
workloads, rounded to bf16 with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

DIR_BITS = (1, 2, 4, 8)


def bf16_round_bits(a: np.ndarray) -> np.ndarray:
    """float32 array -> uint16 bf16 bit patterns, round to nearest even.

    Inputs here are finite; NaN payloads are not preserved.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    rounded = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> float32 (exact widening)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def enabled_dirs(dirs: int) -> list[int]:
    """Direction bit indices (0..3) enabled in a mask, ascending."""
    return [d for d in range(4) if (dirs >> d) & 1]


@dataclass
class Workload:
    """One problem instance.

    ``*_store`` hold what the device receives: float32 arrays for fp32
    workloads, uint16 bf16 bit patterns for bf16 workloads.  ``*_f64`` hold
    the exact same values widened to float64 for the oracle.
    """
    B: int
    C: int
    H: int
    W: int
    dirs: int
    groups: int
    cpw: int
    dtype: str  # "f32" or "bf16"
    x_store: np.ndarray
    w_store: np.ndarray
    lam_store: np.ndarray
    u_store: np.ndarray

    def _f64(self, a: np.ndarray) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a).astype(np.float64)
        return a.astype(np.float64)

    @property
    def x(self) -> np.ndarray:
        return self._f64(self.x_store)

    @property
    def w(self) -> np.ndarray:
        return self._f64(self.w_store)

    @property
    def lam(self) -> np.ndarray:
        return self._f64(self.lam_store)

    @property
    def u(self) -> np.ndarray:
        return self._f64(self.u_store)


def _store(a32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_round_bits(a32)
    if dtype == "f32":
        return np.ascontiguousarray(a32, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def slice_xlu(seed: int, b: int, c: int, H: int, W: int, u_ones: bool = False):
    """float32 (x, lam, u) of one (b, c) slice, each [H][W]."""
    rng = np.random.default_rng([seed, 0, b, c])
    n = H * W
    x = rng.standard_normal(n, dtype=np.float32)
    lam = rng.random(n, dtype=np.float32)
    u = rng.random(n, dtype=np.float32)
    if u_ones:
        u = np.ones(n, dtype=np.float32)
    return x.reshape(H, W), lam.reshape(H, W), u.reshape(H, W)


def slice_w(seed: int, d: int, b: int, k: int, H: int, W: int) -> np.ndarray:
    """float32 raw taps [3][H][W] of direction bit ``d`` for weight set (b, k)."""
    rng = np.random.default_rng([seed, 1, d, b, k])
    return rng.standard_normal(3 * H * W, dtype=np.float32).reshape(3, H, W)


def slice_gy(seed: int, b: int, c: int, H: int, W: int) -> np.ndarray:
    """float32 upstream gradient dL/dy [H][W] of slice (b, c)."""
    rng = np.random.default_rng([seed, 2, b, c])
    return rng.standard_normal(H * W, dtype=np.float32).reshape(H, W)


def make_gy(wl: "Workload", seed: int) -> np.ndarray:
    """Storage-dtype dL/dy [B][C][H][W] for a workload, slice by slice."""
    st = np.uint16 if wl.dtype == "bf16" else np.float32
    gy = np.empty((wl.B, wl.C, wl.H, wl.W), st)
    for b in range(wl.B):
        for c in range(wl.C):
            gy[b, c] = _store(slice_gy(seed, b, c, wl.H, wl.W), wl.dtype)
    return gy


def gy_f64(gy_store: np.ndarray, dtype: str) -> np.ndarray:
    """The exact device values of a stored gradient, widened to float64."""
    return bf16_bits_to_f32(gy_store).astype(np.float64) if dtype == "bf16" else gy_store.astype(np.float64)


def make_workload(B: int, C: int, H: int, W: int, *, dirs: int = 15, groups: int = 1,
                  cpw: int = 1, dtype: str = "bf16", seed: int = 0,
                  u_ones: bool = False) -> Workload:
    """Full seeded workload (every slice), filled slice by slice."""
    if C % cpw:
        raise ValueError("cpw must divide C")
    if dtype not in ("bf16", "f32"):
        raise ValueError(f"unknown dtype {dtype!r}")
    Cw = C // cpw
    ds = enabled_dirs(dirs)
    st = np.uint16 if dtype == "bf16" else np.float32
    x = np.empty((B, C, H, W), st)
    lam = np.empty_like(x)
    u = np.empty_like(x)
    for b in range(B):
        for c in range(C):
            xs, ls, us = slice_xlu(seed, b, c, H, W, u_ones)
            x[b, c], lam[b, c], u[b, c] = _store(xs, dtype), _store(ls, dtype), _store(us, dtype)
    w = np.empty((len(ds), B, Cw, 3, H, W), st)
    for j, d in enumerate(ds):
        for b in range(B):
            for k in range(Cw):
                w[j, b, k] = _store(slice_w(seed, d, b, k, H, W), dtype)
    return Workload(B, C, H, W, dirs, groups, cpw, dtype, x, w, lam, u)


def slice_inputs_f64(seed: int, b: int, c: int, *, H: int, W: int, dirs: int, cpw: int,
                     dtype: str, u_ones: bool = False):
    """Exact device values of one slice, widened to float64.

    Returns (x, w, lam, u) with w of shape [ndir][3][H][W] for weight set
    k = c // cpw.  Matches ``make_workload`` element for element.
    """
    x, lam, u = slice_xlu(seed, b, c, H, W, u_ones)
    ws = np.stack([slice_w(seed, d, b, c // cpw, H, W) for d in enabled_dirs(dirs)])
    out = []
    for a in (x, ws, lam, u):
        s = _store(a, dtype)
        out.append(bf16_bits_to_f32(s).astype(np.float64) if dtype == "bf16" else s.astype(np.float64))
    return tuple(out)


# The five workload shapes the operator is measured and checked on.
CONFIGS = {
    "tiny": dict(B=1, C=8, H=32, W=32, groups=1, cpw=1, dtype="f32", seed=0, u_ones=True),
    "cls56": dict(B=64, C=96, H=56, W=56, groups=1, cpw=1, dtype="bf16", seed=1, u_ones=False),
    "cgspn1k": dict(B=32, C=128, H=64, W=64, groups=1, cpw=8, dtype="bf16", seed=2, u_ones=False),
    "local2k": dict(B=8, C=256, H=128, W=128, groups=8, cpw=1, dtype="bf16", seed=3, u_ones=False),
    "hires512": dict(B=1, C=320, H=512, W=512, groups=1, cpw=1, dtype="bf16", seed=4, u_ones=False),
}


def config_workload(name: str, dirs: int = 15) -> Workload:
    cfg = dict(CONFIGS[name])
    return make_workload(cfg.pop("B"), cfg.pop("C"), cfg.pop("H"), cfg.pop("W"), dirs=dirs, **cfg)


# The 1K C-GSPN block: batch 32, C = 1152 (C-GSPN abstract), projected to a
# 128-channel proxy that the scan runs on (the cgspn1k scan workload).
BLOCK_CONFIGS = {
    "block1k": dict(B=32, C=1152, C_proxy=128, H=64, W=64, groups=1, cpw=8, dtype="bf16", seed=5),
}


class BlockInputs:
    """Seeded inputs of the compressed block in the storage dtype (bf16 bit
    patterns or fp32) and their exact fp64 values.

    x ~ N(0, 1); w_in ~ N(0, 1/C), so that the projected x_proxy, taps,
    lambda and u are of unit scale; w_out ~ N(0, 1/C_proxy).
    """

    def __init__(self, B, C, C_proxy, H, W, *, rows, dirs=15, groups=1, cpw=1, dtype="bf16", seed=0):
        self.B, self.C, self.C_proxy, self.H, self.W = B, C, C_proxy, H, W
        self.dirs, self.groups, self.cpw, self.dtype, self.rows = dirs, groups, cpw, dtype, rows
        rng = np.random.default_rng(seed)
        self.x_store = _store(rng.standard_normal((B, C, H, W), dtype=np.float32), dtype)
        self.w_in_store = _store(rng.standard_normal((rows, C), dtype=np.float32) / np.float32(np.sqrt(C)), dtype)
        self.w_out_store = _store(rng.standard_normal((C, C_proxy), dtype=np.float32) /
                                  np.float32(np.sqrt(C_proxy)), dtype)

    def _f64(self, a):
        return bf16_bits_to_f32(a).astype(np.float64) if self.dtype == "bf16" else a.astype(np.float64)

    def f64(self):
        return self._f64(self.x_store), self._f64(self.w_in_store), self._f64(self.w_out_store)
