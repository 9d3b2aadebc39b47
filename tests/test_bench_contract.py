"""bench.py's contract, checked without a GPU: one GPU only, the committed
profiles recorded from the current kernel sources, and the
algorithmic byte count of the default workload worked out by hand.

cgspn1k: B = 32, C = 128, 64 x 64, cpw = 8, bf16, four directions, one group.
  x, lambda, u read and y written: 4 * 32*128*4096 * 2 B = 134,217,728 B.
  Taps read: per direction and weight set (32 * 16 of them), the 63 lines
  after the first, each with 3 * 64 - 2 existing taps (the two border
  positions miss one each): 4 * 512 * 63 * 190 * 2 B = 49,029,120 B.
  Total 183,246,848 B.
"""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_default_workload_bytes_by_hand():
    assert 4 * 32 * 128 * 4096 * 2 == 134_217_728
    assert 4 * 512 * 63 * 190 * 2 == 49_029_120
    assert bench.algorithmic_bytes(32, 128, 64, 64, 15, 1, 8, "bf16") == 183_246_848


def test_local_groups_and_short_lines_bytes():
    # TB on an 8 x 4 grid in two groups of 4 lines, fp32: the first line of
    # each group reads no taps, so 6 lines of 3 * 4 - 2 taps, for 2 channels
    E = 1 * 2 * 8 * 4
    assert bench.algorithmic_bytes(1, 2, 8, 4, 1, 2, 1, "f32") == 4 * E * 4 + 2 * 6 * 10 * 4
    # LR on a 1 x 5 grid: lines of one position, one tap each, 4 lines after the first
    assert bench.algorithmic_bytes(1, 1, 1, 5, 4, 1, 1, "f32") == 4 * 5 * 4 + 4 * 1 * 4


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_profiles_match_the_kernel_sources():
    # every summary under profiles/ that carries a kernel source hash was
    # recorded from the sources as they stand (bench.py reports no counter
    # traffic for a kernel that changed since its counters were taken)
    import glob
    checked = 0
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt"))):
        recorded = None
        with open(path) as f:
            for line in f:
                if line.startswith("kernel_source_hash:"):
                    recorded = line.split(":", 1)[1].strip()
        if recorded is None:
            continue
        kernel = next(k for k in ("fused_scan_kernel", "fused_bwd_kernel", "slice_scan_kernel")
                      if os.path.basename(path).startswith(k))
        pass_ = "bwd" if kernel == "fused_bwd_kernel" else "fwd"
        assert recorded == bench.kernel_source_hash(pass_, kernel), f"{path} was recorded from other sources"
        checked += 1
    assert checked >= 6
