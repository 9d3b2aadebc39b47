"""Build libgspn.so (HIP, gfx950) in place with hipcc.

    python -m linear_spatial_propagation_amd.build

Every source is compiled for gfx950 only.  Packed-fp32 VALU instructions are
disabled (-packed-fp32-ops); hipcc's host pass warns that it does not know
that feature, which is expected.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgspn.so")
SOURCES = ["gspn_api.hip", "gspn_fused.hip", "gspn_lines.hip", "gspn_lines_bwd.hip", "gspn_fused_bwd.hip",
           "gspn_general.hip", "gspn_block.hip", "gspn_slice.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libgspn.so; returns its path."""
    out_dir = os.path.join(HERE, "_build")
    os.makedirs(out_dir, exist_ok=True)
    objs = []
    for src in SOURCES:
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        cmd = [hipcc(), *flags(), "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {src}")
        objs.append(obj)
    tmp = LIB + f".tmp{os.getpid()}"
    # rocBLAS runs the block's two projections (plain GEMMs)
    rocm_lib = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "lib")
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp, f"-L{rocm_lib}",
           "-lrocblas", f"-Wl,-rpath,{rocm_lib}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("linking libgspn.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
