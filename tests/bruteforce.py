"""Dense closed-form checker for the GSPN line scan (tiny grids only).

An independent formulation used to pin the fp64 oracle.  Per the
"Key design 1: stability-context condition" section of the GSPN (CVPR 2025)
paper notes, unrolling h_i = w_i h_{i-1} + lambda_i x_i gives

    h_i = sum_{j = i0}^{i} W_ij (lambda_j x_j),   W_ij = w_i w_{i-1} ... w_{j+1},
    W_ii = I,

with i0 the first line of the group ("Key design 3": local groups propagate
independently, so the sum starts at the group's first line).  Every w_tau is
built here as a dense m x m matrix from its tridiagonal taps ("Key design 2":
each pixel links to the 3 adjacent pixels of the previous line) and every
W_ij is formed by explicit matrix products.  Theorem 1 of the same section
(row-stochastic factors give unit row sums) is asserted on every W_ij.

The four directions are obtained by flipping/transposing the grid into the
top-to-bottom orientation, scanning, and transforming back -- a different
route from the oracle's per-pixel index mapping.
"""
from __future__ import annotations

import numpy as np


def _to_tb(a: np.ndarray, d: int) -> np.ndarray:
    """[..., H, W] -> the array whose rows are direction d's lines in scan order."""
    if d == 0:
        return a
    if d == 1:
        return a[..., ::-1, :]
    if d == 2:
        return np.swapaxes(a, -1, -2)
    return np.swapaxes(a, -1, -2)[..., ::-1, :]


def _from_tb(a: np.ndarray, d: int) -> np.ndarray:
    if d == 0:
        return a
    if d == 1:
        return a[..., ::-1, :]
    if d == 2:
        return np.swapaxes(a, -1, -2)
    return np.swapaxes(a[..., ::-1, :], -1, -2)


def dense_line_matrix(taps: np.ndarray) -> np.ndarray:
    """taps [3][m] raw values of one line -> dense m x m row-stochastic w_i.

    Row p holds sigmoid(taps[t, p]) / (sum over existing taps) in column
    p + t - 1; taps pointing outside the line do not exist.
    """
    m = taps.shape[1]
    w = np.zeros((m, m))
    for p in range(m):
        cols = [(t, p + t - 1) for t in range(3) if 0 <= p + t - 1 < m]
        sig = np.array([1.0 / (1.0 + np.exp(-taps[t, p])) for t, _ in cols])
        sig = sig / sig.sum()
        for (t, col), v in zip(cols, sig):
            w[p, col] = v
    return w


def scan_tb_dense(xl: np.ndarray, taps: np.ndarray, groups: int, check: bool = True) -> np.ndarray:
    """Closed-form top-to-bottom scan of one slice.

    xl: [n][m] lambda * x in scan orientation; taps: [3][n][m].
    """
    n, m = xl.shape
    L = n // groups
    ws = [dense_line_matrix(taps[:, i, :]) for i in range(n)]
    h = np.zeros((n, m))
    ones = np.ones(m)
    for i in range(n):
        i0 = (i // L) * L
        for j in range(i0, i + 1):
            Wij = np.eye(m)
            for tau in range(j + 1, i + 1):   # W_ij = w_i ... w_{j+1}
                Wij = ws[tau] @ Wij
            if check:
                assert np.allclose(Wij @ ones, ones, rtol=0, atol=1e-12), "Theorem 1 violated"
            h[i] += Wij @ xl[j]
    return h


def bruteforce_fwd(x, w, lam, u, *, dirs: int = 15, groups: int = 1, cpw: int = 1,
                   check: bool = True) -> np.ndarray:
    """y[B][C][H][W] by the dense closed form.  Same tensor layouts as the oracle.

    lam and u may also carry a leading direction axis ([ndir][B][C][H][W]):
    then direction d is driven by its own lam_d and y = sum_d u_d h_d.
    """
    x, w, lam, u = (np.asarray(a, dtype=np.float64) for a in (x, w, lam, u))
    B, C, H, W = x.shape
    y = np.zeros_like(x)
    for b in range(B):
        for c in range(C):
            acc = np.zeros((H, W))
            slab = 0
            for d in range(4):
                if not (dirs >> d) & 1:
                    continue
                taps = w[slab, b, c // cpw]          # [3][H][W]
                lam_bc = lam[slab, b, c] if lam.ndim == 5 else lam[b, c]
                gate = u[slab, b, c] if u.ndim == 5 else np.ones((H, W))
                slab += 1
                xl = _to_tb(lam_bc * x[b, c], d)
                h = scan_tb_dense(xl, _to_tb(taps, d), groups, check)
                acc += gate * _from_tb(h, d)
            y[b, c] = acc if u.ndim == 5 else u[b, c] * acc
    return y
