"""ctypes binding of libgspn.so (the C ABI declared in include/gspn.h).

Argument marshalling only: every step of the operator runs in the HIP
kernels of the shared library.  If the library is missing this module raises;
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgspn.so")

GSPN_F32 = 0
GSPN_BF16 = 1
PATH_AUTO = 0
PATH_FUSED = 1
PATH_GENERAL = 2
PATH_SLICE = 3
DIR_TB, DIR_BT, DIR_LR, DIR_RL, DIR_ALL = 1, 2, 4, 8, 15

LAM_PER_DIR, U_PER_DIR = 1, 2
MAX_BATCH = 32
NOALLOC_SCRATCH_BYTES = 64 << 20
BLOCK_RMSNORM = 1
ERR_SCRATCH = -12


class Problem(ctypes.Structure):
    """gspn_problem of include/gspn.h."""
    _fields_ = [("x", ctypes.c_void_p), ("w_raw", ctypes.c_void_p), ("lam", ctypes.c_void_p),
                ("u", ctypes.c_void_p), ("y", ctypes.c_void_p), ("B", ctypes.c_int64),
                ("C", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
                ("dirs", ctypes.c_uint32), ("groups", ctypes.c_int32), ("ch_per_weight", ctypes.c_int32)]

EXPORTED = ("gspn_scan_fwd", "gspn_scan_fwd_noalloc", "gspn_scan_fwd_path", "gspn_scan_fwd_ex", "gspn_scan_fwd_batched",
            "gspn_select_path", "gspn_scan_bwd",
            "gspn_scan_bwd_path", "gspn_scan_bwd_ex", "gspn_bwd_supported", "gspn_block_fwd", "gspn_block_rows",
            "gspn_status_string", "gspn_last_error", "gspn_version")

_lock = threading.Lock()
_lib = None


class GspnError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(text)
        self.status = status


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libgspn.so once; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with "
                               "`python -m linear_spatial_propagation_amd.build`")
        lib = ctypes.CDLL(path)
        vp, i64, u32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_int32
        lib.gspn_scan_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, u32, i32, i32, i32, vp]
        lib.gspn_scan_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, u32, i32, i32, i32, vp]
        lib.gspn_scan_fwd_noalloc.restype = ctypes.c_int
        lib.gspn_scan_fwd.restype = ctypes.c_int
        lib.gspn_scan_fwd_path.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, u32, i32, i32, i32,
                                           i32, vp]
        lib.gspn_scan_fwd_path.restype = ctypes.c_int
        lib.gspn_scan_fwd_ex.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, u32, i32, i32, u32, i32, vp]
        lib.gspn_scan_fwd_ex.restype = ctypes.c_int
        lib.gspn_scan_fwd_batched.argtypes = [ctypes.POINTER(Problem), i32, i32, vp]
        lib.gspn_scan_fwd_batched.restype = ctypes.c_int
        lib.gspn_select_path.argtypes = [i64, i64, i64, i64, u32, i32, i32, i32]
        lib.gspn_select_path.restype = ctypes.c_int
        lib.gspn_scan_bwd.argtypes = [vp] * 9 + [i64, i64, i64, i64, u32, i32, i32, i32, vp]
        lib.gspn_scan_bwd.restype = ctypes.c_int
        lib.gspn_scan_bwd_path.argtypes = [vp] * 9 + [i64, i64, i64, i64, u32, i32, i32, i32, i32, vp]
        lib.gspn_scan_bwd_path.restype = ctypes.c_int
        lib.gspn_scan_bwd_ex.argtypes = [vp] * 9 + [i64, i64, i64, i64, u32, i32, i32, u32, i32, vp]
        lib.gspn_scan_bwd_ex.restype = ctypes.c_int
        lib.gspn_bwd_supported.argtypes = [i64, i64, i64, i64, u32, i32, i32, i32]
        lib.gspn_bwd_supported.restype = ctypes.c_int
        lib.gspn_block_fwd.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64, u32, i32, i32, u32, i32, vp]
        lib.gspn_block_fwd.restype = ctypes.c_int
        lib.gspn_block_rows.argtypes = [i64, u32, i32]
        lib.gspn_block_rows.restype = ctypes.c_int64
        lib.gspn_status_string.argtypes = [ctypes.c_int]
        lib.gspn_status_string.restype = ctypes.c_char_p
        lib.gspn_last_error.argtypes = []
        lib.gspn_last_error.restype = ctypes.c_char_p
        lib.gspn_version.argtypes = []
        lib.gspn_version.restype = ctypes.c_int
        _lib = lib
        return lib


def status_string(status: int) -> str:
    return load().gspn_status_string(status).decode()


def check(status: int) -> None:
    if status != 0:
        lib = load()
        detail = lib.gspn_last_error().decode()
        msg = lib.gspn_status_string(status).decode()
        raise GspnError(status, msg + (f" [{detail}]" if detail else ""))


def scan_fwd_ptr(x: int, w: int, lam: int, u: int, y: int, B: int, C: int, H: int, W: int, *,
                 dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1, dtype: int = GSPN_BF16,
                 path: int = PATH_AUTO, stream: int = 0) -> int:
    """Raw call on device pointers; returns the status code."""
    return load().gspn_scan_fwd_path(x, w, lam, u, y, B, C, H, W, dirs, groups, ch_per_weight,
                                     dtype, path, stream)


def scan_fwd_noalloc_ptr(x: int, w: int, lam: int, u: int, y: int, B: int, C: int, H: int, W: int, *,
                         dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1, dtype: int = GSPN_BF16,
                         stream: int = 0) -> int:
    """Raw call of the allocation-free forward on device pointers; returns the status code."""
    return load().gspn_scan_fwd_noalloc(x, w, lam, u, y, B, C, H, W, dirs, groups, ch_per_weight, dtype, stream)


def scan_fwd_ex_ptr(x: int, w: int, lam: int, u: int, y: int, B: int, C: int, H: int, W: int, *,
                    dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1, flags: int = 0,
                    dtype: int = GSPN_BF16, stream: int = 0) -> int:
    """Raw call of the per-direction variant on device pointers; returns the status code."""
    return load().gspn_scan_fwd_ex(x, w, lam, u, y, B, C, H, W, dirs, groups, ch_per_weight, flags,
                                   dtype, stream)


def scan_fwd_batched_ptr(problems, dtype: int = GSPN_BF16, stream: int = 0) -> int:
    """Raw batched call: `problems` is a sequence of Problem; returns the status code."""
    arr = (Problem * max(1, len(problems)))(*problems)
    return load().gspn_scan_fwd_batched(arr, len(problems), dtype, stream)


def scan_bwd_ptr(x: int, w: int, lam: int, u: int, gy: int, gx: int, gw: int, glam: int, gu: int,
                 B: int, C: int, H: int, W: int, *, dirs: int = DIR_ALL, groups: int = 1,
                 ch_per_weight: int = 1, dtype: int = GSPN_BF16, path: int = PATH_AUTO,
                 stream: int = 0) -> int:
    """Raw backward call on device pointers; returns the status code."""
    return load().gspn_scan_bwd_path(x, w, lam, u, gy, gx, gw, glam, gu, B, C, H, W, dirs, groups,
                                     ch_per_weight, dtype, path, stream)


def scan_bwd_ex_ptr(x: int, w: int, lam: int, u: int, gy: int, gx: int, gw: int, glam: int, gu: int,
                    B: int, C: int, H: int, W: int, *, dirs: int = DIR_ALL, groups: int = 1,
                    ch_per_weight: int = 1, flags: int = 0, dtype: int = GSPN_BF16, stream: int = 0) -> int:
    """Raw backward of the per-direction variant on device pointers; returns the status code."""
    return load().gspn_scan_bwd_ex(x, w, lam, u, gy, gx, gw, glam, gu, B, C, H, W, dirs, groups,
                                   ch_per_weight, flags, dtype, stream)


def bwd_supported(B, C, H, W, *, dirs=DIR_ALL, groups=1, ch_per_weight=1, dtype=GSPN_BF16) -> int:
    return load().gspn_bwd_supported(B, C, H, W, dirs, groups, ch_per_weight, dtype)


def select_path(B, C, H, W, *, dirs=DIR_ALL, groups=1, ch_per_weight=1, dtype=GSPN_BF16) -> int:
    return load().gspn_select_path(B, C, H, W, dirs, groups, ch_per_weight, dtype)


def block_fwd_ptr(x: int, w_in: int, w_out: int, z: int, B: int, C: int, C_proxy: int, H: int, W: int, *,
                  dirs: int = DIR_ALL, groups: int = 1, ch_per_weight: int = 1, flags: int = 1,
                  dtype: int = GSPN_BF16, stream: int = 0) -> int:
    """Raw call of the compressed block on device pointers; returns the status code."""
    return load().gspn_block_fwd(x, w_in, w_out, z, B, C, C_proxy, H, W, dirs, groups, ch_per_weight, flags,
                                 dtype, stream)


def block_rows(C_proxy: int, dirs: int = DIR_ALL, ch_per_weight: int = 1) -> int:
    """Rows of the block's input projection (or a negative status code)."""
    return load().gspn_block_rows(C_proxy, dirs, ch_per_weight)
