#!/usr/bin/env python3
"""Benchmark of the GSPN 4-direction line-scan forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config cgspn1k] [--pass fwd|bwd]

One step = one call of gspn_scan_fwd (the whole forward: weight
normalisation, the four directional scans, merge and store) over one batch
of seeded synthetic inputs already resident in HBM.  The default workload is
the compressed C-GSPN 1K block operator: B=32, C=128 (the propagation
dimension projected from 1152), a 64 x 64 token grid, one weight map per 8
channels, bf16 I/O with fp32 arithmetic, all four directions.

Timing: W untimed warm-up steps, then K timed steps between two device
synchronisations.  The steps rotate over R input/output buffer sets whose
total footprint exceeds 512 MB, so the 256 MB Infinity Cache cannot serve a
step's inputs from the previous step; a same-buffer ("hot") figure is
reported separately.  The K timed steps run back to back (the throughput
`value`).  Then a roofline pass, whose length does not depend on K: 20 more
untimed steps, then 200 steps each bracketed by HIP events on the stream the
kernels run on; roofline.achieved is the algorithmic bytes over the median
of those 200 durations.  `--profile-run` stops after the roofline pass (no
hot pass, copy or CPU leg), and `--summarize-trace` turns the rocprofv3
kernel trace of such a run into the committed kernel-time summary over the
same 200 steps.  The plain forward and backward steps call the C ABI
directly with argument tuples built once.

device_copy_gbps: a plain 512 MiB device-to-device copy on the same GPU
(read + write bytes per second), the practical streaming ceiling, for context.

other_workloads: the forward of every other workload (fused, slice or line
kernels, as the library picks), each with its backward (`bwd`); backward: the
default workload's backward.  Device-drawn inputs of the workloads'
distributions, back-to-back calls on one buffer set; reported beside the
headline, not part of it.

value = algorithmic bytes x K / elapsed time (GB/s, 1e9 B/s).  Algorithmic
bytes count each input once, y once, and only the taps the method consumes:
    s * (|x| + |lam| + |u| + |y|) + s * B * Cw * sum_d (n_d - g) * (3 m_d - 2)
(group-start lines and taps past a line border are never read).

With --pass bwd a step is one call of gspn_scan_bwd instead (the backward:
forward states recomputed, adjoint scans, all four gradients), and its
algorithmic bytes are the inputs x, lam, u, gy once, the taps the forward
consumes, gx, glam, gu once and the whole tap-gradient tensor once:
    s * (4 + 3) * |x| + s * B * Cw * sum_d (n_d - g) * (3 m_d - 2)
    + s * ndir * B * Cw * 3 * H * W.
Its roofline object covers the whole call (all of its launches).

With --batched K (grids up to 64 x 64) a step is one gspn_scan_fwd_batched
call over K copies of the workload (own buffers each), and the same K
problems are also timed as K separate gspn_scan_fwd calls for comparison.

With --variant dirs a step is one call of gspn_scan_fwd_ex with lambda and
u per direction (y = sum_d u_d * h_d); the algorithmic bytes count the four
lambda and four u slabs once:
    s * (|x| + ndir |lam| + ndir |u| + |y|) + (taps as for the forward).
With --pass bwd --variant dirs a step is one call of gspn_scan_bwd_ex (the
backward of that variant); lambda, u and their gradients count ndir slabs:
    (the backward's bytes) + s * 4 * (ndir - 1) * |x|.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GSPN scan GB/s and % of HBM peak (4-dir fwd), 1K C-GSPN config"
METRIC_BWD = "GSPN scan backward GB/s and % of HBM peak (4-dir bwd)"
METRIC_DIRS = "GSPN scan GB/s and % of HBM peak (4-dir fwd, per-direction lambda and u)"
METRIC_BWD_DIRS = "GSPN scan backward GB/s and % of HBM peak (4-dir bwd, per-direction lambda and u)"
HBM_PEAK_GBPS = 8000.0
# steady-state pass after the timed region: untimed steps, then steps back to back
ROOF_WARM, ROOF_N = 20, 200
HOT_N = 50
COPY_CALIBRATION_BYTES = 256 * 1024 * 1024
# The dominant kernel of each pass on the default workload (C-GSPN 1K, 64 x 64
# grids: one fused kernel per call), the sources its code comes from, and its
# committed rocprofv3 summaries.
PASSES = {
    "fwd": {"kernel": "fused_scan_kernel",
            "sources": ["linear_spatial_propagation_amd/csrc/gspn_fused.hip",
                        "linear_spatial_propagation_amd/csrc/gspn_device.h"]},
    "bwd": {"kernel": "fused_bwd_kernel",
            "sources": ["linear_spatial_propagation_amd/csrc/gspn_fused_bwd.hip",
                        "linear_spatial_propagation_amd/csrc/gspn_lines.h",
                        "linear_spatial_propagation_amd/csrc/gspn_device.h"]},
}


def profile_path(pass_, what, config="cgspn1k"):
    return os.path.join(ROOT, "profiles", f"{PASSES[pass_]['kernel']}_{config}_{what}.txt")


def algorithmic_bytes(B, C, H, W, dirs, groups, cpw, dtype) -> int:
    s = 2 if dtype == "bf16" else 4
    E = B * C * H * W
    total = 4 * E * s
    Cw = C // cpw
    for d in range(4):
        if (dirs >> d) & 1:
            n, m = (H, W) if d < 2 else (W, H)
            total += s * B * Cw * (n - groups) * max(3 * m - 2, 1 if m == 1 else 0)
    return total


def algorithmic_bytes_bwd(B, C, H, W, dirs, groups, cpw, dtype) -> int:
    s = 2 if dtype == "bf16" else 4
    E = B * C * H * W
    nd = bin(dirs & 15).count("1")
    fwd_taps = algorithmic_bytes(B, C, H, W, dirs, groups, cpw, dtype) - 4 * E * s
    return 7 * E * s + fwd_taps + s * nd * B * (C // cpw) * 3 * H * W


# sources of the kernels whose counter summaries carry a source hash
KERNEL_SOURCES = {
    "slice_scan_kernel": ["linear_spatial_propagation_amd/csrc/gspn_slice.hip",
                          "linear_spatial_propagation_amd/csrc/gspn_device.h"],
}


def kernel_source_hash(pass_="fwd", kernel=None) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel] if kernel in KERNEL_SOURCES else PASSES[pass_]["sources"]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _read_summary(path):
    out = {}
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("#") or ":" not in line:
                    continue
                k, v = line.split(":", 1)
                out[k.strip()] = v.strip()
    except OSError:
        pass
    return out


def load_traffic(pass_="fwd", kernel=None, config="cgspn1k"):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    `kernel` (default: the pass's fused kernel) on `config`, or None when there
    is none or the kernel source changed since the counters were taken."""
    kernel = kernel or PASSES[pass_]["kernel"]
    t = _read_summary(os.path.join(ROOT, "profiles", f"{kernel}_{config}_traffic.txt"))
    if t.get("kernel_source_hash") != kernel_source_hash(pass_, kernel):
        return None
    try:
        return int(float(t["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _kernel_short(name):
    """Short kernel name (the template arguments dropped)."""
    for k in ("fused_scan_batched_kernel", "fused_scan_kernel", "slice_scan_kernel", "fused_bwd_kernel",
              "adjoint_scan_kernel",
              "line_scan_kernel", "transpose_kernel", "convert_kernel", "merge_dirs_kernel", "merge_kernel",
              "direction_kernel", "outproj_kernel", "rms_scale_kernel"):
        if k in name:
            return k
    if "copyBuffer" in name:
        return "copy"
    return name[:48]


def summarize_pmc(pmc_dir, command, config="cgspn1k", pass_="fwd", name=None):
    """Summarise two rocprofv3 --pmc passes (FETCH_SIZE, WRITE_SIZE) of a bench
    run with --copy-calibration into the traffic summary under profiles/.

    FETCH_SIZE / WRITE_SIZE are KiB per dispatch.  Each is scaled by the
    ratio between the known size of the plain device copy (256 MiB read,
    256 MiB written) and what the same counter reads for that copy.  A step
    may run several of the library's kernels (the line path); the bytes of
    one step are the sum over its dispatches, and the number of steps is the
    number of dispatches of the step's anchor kernel (run once per step)."""
    import csv
    import glob
    from linear_spatial_propagation_amd.inputs import CONFIGS
    per = {}
    for f in glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            key = (row["Counter_Name"], int(row["Dispatch_Id"]))
            per.setdefault(key, [row["Kernel_Name"], 0.0])
            per[key][1] += float(row["Counter_Value"])
    vals = {}
    for (counter, did), (kname_full, v) in per.items():
        short = "copy" if "copyBuffer" in kname_full else (
            _kernel_short(kname_full) if any(k in kname_full for k in GSPN_KERNELS) else None)
        if short:
            vals.setdefault((counter, short), []).append((did, v))
    copy_w = max(v for _, v in vals[("WRITE_SIZE", "copy")])
    copy_w_id = [d for d, v in vals[("WRITE_SIZE", "copy")] if v == copy_w][0]
    copy_f = dict(vals[("FETCH_SIZE", "copy")]).get(copy_w_id)
    if copy_f is None:   # separate runs number dispatches identically
        copy_f = max(v for _, v in vals[("FETCH_SIZE", "copy")])
    copy_kib = COPY_CALIBRATION_BYTES / 1024
    f_scale, w_scale = copy_kib / copy_f, copy_kib / copy_w
    c = CONFIGS[config]
    kernels = sorted({k for (_, k) in vals if k != "copy"})
    # the kernel run once per step: the single-kernel paths' only kernel, else the line scan
    anchor = next(k for k in ("fused_scan_kernel", "slice_scan_kernel", "fused_bwd_kernel", "line_scan_kernel",
                              "adjoint_scan_kernel") if k in kernels)
    single = anchor in ("fused_scan_kernel", "slice_scan_kernel", "fused_bwd_kernel")
    steps = len(vals[("FETCH_SIZE", anchor)])
    fetch_kib = sum(v for k in kernels for _, v in vals.get(("FETCH_SIZE", k), [])) / steps
    write_kib = sum(v for k in kernels for _, v in vals.get(("WRITE_SIZE", k), [])) / steps
    hbm = fetch_kib * 1024 * f_scale + write_kib * 1024 * w_scale
    alg = (algorithmic_bytes_bwd if pass_ == "bwd" else algorithmic_bytes)(
        c["B"], c["C"], c["H"], c["W"], 15, c["groups"], c["cpw"], c["dtype"])
    lines = [
        f"# rocprofv3 memory counters: {pass_} step on {config} "
        f"(B={c['B']} C={c['C']} H={c['H']} W={c['W']} groups={c['groups']} ch_per_weight={c['cpw']} {c['dtype']})",
        f"# command (two passes, FETCH_SIZE then WRITE_SIZE): {command}",
        "# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; a step's bytes are the sum over its dispatches;",
        "# each is scaled by (known bytes / counter bytes) of a 256 MiB device-to-device copy in the same run.",
    ]
    if single:
        lines.append(f"kernel_source_hash: {kernel_source_hash(pass_, anchor)}")
    lines += [f"steps: {steps}", f"kernels_per_step: {', '.join(kernels)}"]
    for k in kernels:
        fk = sum(v for _, v in vals.get(("FETCH_SIZE", k), [])) / steps
        wk = sum(v for _, v in vals.get(("WRITE_SIZE", k), [])) / steps
        lines.append(f"  {k}: read {fk * 1024 * f_scale / 1e6:.1f} MB, write {wk * 1024 * w_scale / 1e6:.1f} MB per step")
    lines += [
        f"fetch_kib_per_step: {fetch_kib:.1f}",
        f"write_kib_per_step: {write_kib:.1f}",
        f"copy_known_bytes: {COPY_CALIBRATION_BYTES}",
        f"copy_fetch_kib: {copy_f:.1f}",
        f"copy_write_kib: {copy_w:.1f}",
        f"fetch_scale: {f_scale:.4f}",
        f"write_scale: {w_scale:.4f}",
        f"hbm_read_bytes_per_launch: {fetch_kib * 1024 * f_scale:.0f}",
        f"hbm_write_bytes_per_launch: {write_kib * 1024 * w_scale:.0f}",
        f"hbm_bytes_per_launch: {hbm:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {hbm / alg:.4f}",
    ]
    stem = name or (anchor if single else PASSES[pass_]["kernel"])
    with open(os.path.join(ROOT, "profiles", f"{stem}_{config}_traffic.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def summarize_stats(stats_csv, command, config="cgspn1k", pass_="fwd", name=None):
    """Copy the kernel rows of a rocprofv3 --kernel-trace --stats CSV into the
    stats summary under profiles/ (named for `name`, default the pass's
    dominant kernel on the default workload)."""
    import csv
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# rocprofv3 --kernel-trace --stats summary, workload {config}",
             f"# command: {command}",
             "kernel, calls, total_ns, average_ns, min_ns, max_ns, percent"]
    for r in rows:
        lines.append(f"{_kernel_short(r['Name'])}, {r['Calls']}, {r['TotalDurationNs']}, "
                     f"{float(r['AverageNs']):.1f}, {r['MinNs']}, {r['MaxNs']}, {float(r['Percentage']):.2f}")
    out = profile_path(pass_, "stats", config)
    if name:
        out = os.path.join(ROOT, "profiles", f"{name}_{config}_stats.txt")
    else:
        lines.append(f"kernel_source_hash: {kernel_source_hash(pass_)}")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


GSPN_KERNELS = ("fused_scan_kernel", "fused_scan_batched_kernel", "slice_scan_kernel", "fused_bwd_kernel",
                "adjoint_scan_kernel",
                "line_scan_kernel", "transpose_kernel", "convert_kernel", "merge_kernel", "merge_dirs_kernel",
                "direction_kernel", "outproj_kernel", "rms_scale_kernel")


def summarize_trace(trace_csv, command, config, pass_, warmup, steps, name=None):
    """Kernel-time summary of a `--profile-run` bench under rocprofv3
    --kernel-trace: the library's dispatches of the timed region (the K steps
    after the W warm-up steps, whose event-timed average gives
    roofline.achieved), per kernel and per step, and of the steady-state
    pass that follows it."""
    import csv
    import numpy as np
    from linear_spatial_propagation_amd.inputs import CONFIGS
    rows = [r for r in csv.DictReader(open(trace_csv))
            if any(k in r["Kernel_Name"] for k in GSPN_KERNELS)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    total_steps = warmup + steps + ROOF_WARM + ROOF_N
    if len(rows) % total_steps:
        raise SystemExit(f"{len(rows)} library dispatches do not divide into {total_steps} steps")
    per_step = len(rows) // total_steps
    c = CONFIGS[config]
    alg = (algorithmic_bytes_bwd if pass_ == "bwd" else algorithmic_bytes)(
        c["B"], c["C"], c["H"], c["W"], 15, c["groups"], c["cpw"], c["dtype"])
    lines = [f"# rocprofv3 --kernel-trace summary, workload {config} ({pass_}); {per_step} library dispatch(es) "
             "per step",
             f"# timed region: steps {warmup}..{warmup + steps - 1} (after {warmup} warm-up steps); steady state: "
             f"the {ROOF_N} steps after {ROOF_WARM} more untimed ones",
             f"# command: {command}"]

    def part(label, first, count):
        sel = rows[first * per_step:(first + count) * per_step]
        dur = np.array([int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in sel], dtype=np.float64)
        span = (int(sel[-1]["End_Timestamp"]) - int(sel[0]["Start_Timestamp"])) / count
        step_ns = dur.reshape(count, per_step).sum(axis=1)
        names = [_kernel_short(r["Kernel_Name"]) for r in sel]
        out = [f"[{label}] kernel, dispatches, average_ns, median_ns, min_ns, max_ns"]
        for k in dict.fromkeys(names):
            d = np.array([v for v, n in zip(dur, names) if n == k])
            out.append(f"{k}, {len(d)}, {d.mean():.1f}, {np.median(d):.1f}, {d.min():.0f}, {d.max():.0f}")
        avg = float(step_ns.mean())
        out += [f"{label}_step_kernel_ns_average: {avg:.1f}",
                f"{label}_step_kernel_ns_median: {np.median(step_ns):.1f}",
                f"{label}_first_start_to_last_end_ns_per_step: {span:.1f}",
                f"{label}_achieved_gbps_at_average: {alg / avg:.1f}",
                f"{label}_frac_of_8000_gbps_at_average: {alg / avg / HBM_PEAK_GBPS:.4f}"]
        return out

    lines += part("timed", warmup, steps)
    lines += part("steady", warmup + steps + ROOF_WARM, ROOF_N)
    lines.append(f"algorithmic_bytes_per_step: {alg}")
    if name is None:
        # a step that is one kernel is summarised under that kernel's name,
        # with the hash of the source it was built from
        kinds = set(_kernel_short(r["Kernel_Name"]) for r in rows)
        if len(kinds) != 1:
            raise SystemExit(f"kernels {sorted(kinds)} in one step: give --profile-name")
        name = kinds.pop()
        if name in KERNEL_SOURCES or name == PASSES[pass_]["kernel"]:
            lines.append(f"kernel_source_hash: {kernel_source_hash(pass_, name)}")
    stem = name
    out = os.path.join(ROOT, "profiles", f"{stem}_{config}_stats.txt")
    with open(out, "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg_name: str, budget_s: float = 4.0, backward: bool = False):
    """Time the fp64 oracle, as it stands, on a bounded sample of the same
    workload: whole batch items.  Three runs with every thread the oracle
    gets (each repeats the sample for about budget_s seconds; the median run
    is the value), then three runs on one thread over a smaller sample."""
    import numpy as np
    import oracle
    from linear_spatial_propagation_amd.inputs import CONFIGS, gy_f64, make_gy, make_workload

    cfg = dict(CONFIGS[cfg_name])
    B = cfg.pop("B")
    C, H, W = cfg.pop("C"), cfg.pop("H"), cfg.pop("W")
    threads = oracle.max_threads()

    def prepare(nb):
        wl = make_workload(nb, C, H, W, **cfg)
        args = (wl.x, wl.w, wl.lam, wl.u)
        if backward:
            args += (gy_f64(make_gy(wl, 1000 + cfg["seed"]), wl.dtype),)
        return wl, args

    def once(wl, args, nthreads):
        t0 = time.perf_counter()
        fn = oracle.scan_bwd if backward else oracle.scan_fwd
        fn(*args, dirs=15, groups=wl.groups, cpw=wl.cpw, nthreads=nthreads)
        return time.perf_counter() - t0

    def rate(nb, nthreads, t_single):
        """Median over three runs of GB/s; each run repeats the sample for
        about budget_s / 3 seconds."""
        wl, args = prepare(nb)
        nbytes = (algorithmic_bytes_bwd if backward else algorithmic_bytes)(
            nb, C, H, W, 15, cfg["groups"], cfg["cpw"], cfg["dtype"])
        reps = max(1, int(budget_s / 3 / max(t_single, 1e-6)))
        runs = []
        for _ in range(3):
            t = sum(once(wl, args, nthreads) for _ in range(reps)) / reps
            runs.append(nbytes / t / 1e9)
        return float(np.median(runs)), reps

    wl1, args1 = prepare(1)
    t1 = once(wl1, args1, threads)                  # one batch item, every thread
    nb = int(max(1, min(B, budget_s / 6 / max(t1, 1e-6))))
    all_threads, reps = rate(nb, threads, t1 * nb)
    t1s = once(wl1, args1, 1)                       # one batch item, one thread
    nb1 = int(max(1, min(B, budget_s / 6 / max(t1s, 1e-6))))
    one_thread, reps1 = rate(nb1, 1, t1s * nb1)
    return {"value": round(all_threads, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "one_thread_value": round(one_thread, 4),
            "sample": f"{nb} of {B} batch items ({nb * C} (b,c) slices) of the same workload, fp64 C oracle "
                      f"with OpenMP over slices on {threads} threads, median of 3 runs of {reps} repeats; "
                      f"one thread: {nb1} batch item(s), median of 3 runs of {reps1} repeats"}


def bench_block(args):
    """The compressed block on the 1K block workload: tokens per second.

    One step is one gspn_block_fwd call: the input projection (rocBLAS), the
    scan (libgspn kernels), the output projection with the RMS normalisation
    fused into it (a libgspn MFMA kernel).  The roofline
    counts the bytes no implementation can avoid (x read, z written, both
    weight matrices read once) against HBM; the GEMM rate is reported
    beside it.
    """
    import numpy as np
    import torch

    import linear_spatial_propagation_amd as gspn
    from linear_spatial_propagation_amd.inputs import BLOCK_CONFIGS, BlockInputs

    cfg = dict(BLOCK_CONFIGS["block1k"])
    seed = cfg.pop("seed")
    B, C, Cp, H, W = cfg.pop("B"), cfg.pop("C"), cfg.pop("C_proxy"), cfg.pop("H"), cfg.pop("W")
    rows = gspn.block_rows(Cp, ch_per_weight=cfg["cpw"])
    inp = BlockInputs(B, C, Cp, H, W, rows=rows, seed=seed, **cfg)
    dev = torch.device("cuda:0")

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if inp.dtype == "bf16" else t).to(dev)

    x, wi, wo = up(inp.x_store), up(inp.w_in_store), up(inp.w_out_store)
    z = torch.empty_like(x)
    stream = torch.cuda.current_stream(dev)

    def step():
        gspn.block_fwd(x, wi, wo, groups=inp.groups, ch_per_weight=inp.cpw, out=z)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize(dev)
    elapsed = time.perf_counter() - t0
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(args.steps, 50))]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize(dev)
    per = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    es = 2 if inp.dtype == "bf16" else 4
    HW = H * W
    nbytes = (2 * B * C * HW + rows * C + C * Cp) * es
    flops = 2 * B * HW * C * (rows + Cp)
    med = float(np.median(per))
    out = {
        "metric": "C-GSPN compressed block forward, tokens/s (projection, scan, RMS normalisation fused into the projection back)",
        "value": round(B * HW * args.steps / elapsed, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 GEMM inputs, fp32 accumulation; fp32 scan arithmetic",
        "data": "synthetic",
        "config": {"workload": f"block1k: B={B} C={C} C_proxy={Cp} H={H} W={W} groups={inp.groups} "
                               f"ch_per_weight={inp.cpw} dirs=TB|BT|LR|RL, {inp.dtype} I/O",
                   "w_in_rows": rows, "seed": seed},
        "launch_us": {"median": round(med * 1e6, 2), "p10": round(float(np.percentile(per, 10)) * 1e6, 2),
                      "p90": round(float(np.percentile(per, 90)) * 1e6, 2)},
        "gemm_tflops_at_median": round(flops / med / 1e12, 1),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / med / 1e9, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(nbytes / med / 1e9 / HBM_PEAK_GBPS, 4), "traffic": None,
                     "kernel": "gspn_block_fwd, all launches of one call (x, z and the weights once)"},
    }
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="cgspn1k")
    ap.add_argument("--pass", dest="pass_", choices=("fwd", "bwd"), default="fwd",
                    help="time the forward (default) or the backward")
    ap.add_argument("--variant", choices=("none", "dirs"), default="none",
                    help="dirs: per-direction lambda and u (gspn_scan_fwd_ex; with --pass bwd, gspn_scan_bwd_ex)")
    ap.add_argument("--batched", type=int, default=1,
                    help="K > 1: K copies of the workload in one batched launch (gspn_scan_fwd_batched)")
    ap.add_argument("--block", action="store_true",
                    help="time the compressed block (gspn_block_fwd) on the 1K block workload")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-others", dest="others", action="store_false",
                    help="skip the forward timing of the other workloads (the other_workloads object)")
    ap.add_argument("--profile-run", action="store_true",
                    help="warm-up, timed steps and the roofline pass only (no hot pass, copy or CPU leg): "
                         "the run a kernel-trace summary is taken from")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 256 MiB device copy (for counter calibration)")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="write the traffic summary from rocprofv3 --pmc output in DIR and exit")
    ap.add_argument("--profile-name", default=None,
                    help="file-name stem of the --summarize-stats summary (default: the dominant kernel)")
    ap.add_argument("--summarize-stats", metavar="CSV",
                    help="write the kernel-time summary from a rocprofv3 --stats CSV and exit")
    ap.add_argument("--profile-command", default="", help="command line recorded in the summary")
    ap.add_argument("--summarize-trace", metavar="CSV",
                    help="write the kernel-time summary of a --profile-run from its rocprofv3 kernel-trace CSV "
                         "(give the run's --steps and --warmup) and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc, args.profile_command, args.config, args.pass_, args.profile_name)
        return
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.profile_command, args.config, args.pass_, args.warmup,
                        args.steps, args.profile_name)
        return
    if args.summarize_stats:
        summarize_stats(args.summarize_stats, args.profile_command, args.config, args.pass_,
                        args.profile_name)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the operator has no cross-GPU step, so "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    if args.block:
        bench_block(args)
        return

    import numpy as np
    import torch

    import linear_spatial_propagation_amd as gspn
    from linear_spatial_propagation_amd.inputs import CONFIGS, config_workload

    torch.cuda.init()
    dev = torch.device("cuda:0")
    cfgd = CONFIGS[args.config]
    wl = config_workload(args.config)
    B, C, H, W = wl.B, wl.C, wl.H, wl.W
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    def up(a):
        t = torch.from_numpy(np.ascontiguousarray(a))
        return (t.view(torch.bfloat16) if wl.dtype == "bf16" else t).to(dev)

    bwd = args.pass_ == "bwd"
    dirs_variant = args.variant == "dirs" and not bwd
    bwd_variant = args.variant == "dirs" and bwd
    batched = args.batched if not bwd and not dirs_variant else 1
    base = [up(a) for a in (wl.x_store, wl.w_store, wl.lam_store, wl.u_store)]
    if dirs_variant:
        # per-direction lambda and u: U(0, 1), seeded, in the workload's dtype
        from linear_spatial_propagation_amd.inputs import _store
        rng = np.random.default_rng([cfgd["seed"], 5])
        for i in (2, 3):
            base[i] = up(_store(rng.random((4, B, C, H, W), dtype=np.float32), wl.dtype))
        E0 = B * C * H * W
        nbytes = algorithmic_bytes(B, C, H, W, 15, wl.groups, wl.cpw, wl.dtype) + 6 * E0 * (2 if wl.dtype == "bf16" else 4)
        outs_like = [base[0]]
    elif bwd:
        from linear_spatial_propagation_amd.inputs import make_gy
        base.append(up(make_gy(wl, 1000 + cfgd["seed"])))
        nbytes = algorithmic_bytes_bwd(B, C, H, W, 15, wl.groups, wl.cpw, wl.dtype)
        if bwd_variant:
            from linear_spatial_propagation_amd.inputs import _store
            rng = np.random.default_rng([cfgd["seed"], 5])
            for i in (2, 3):
                base[i] = up(_store(rng.random((4, B, C, H, W), dtype=np.float32), wl.dtype))
            nbytes += 4 * 3 * B * C * H * W * (2 if wl.dtype == "bf16" else 4)
        outs_like = [base[0], base[1], base[2], base[3]]
    else:
        nbytes = algorithmic_bytes(B, C, H, W, 15, wl.groups, wl.cpw, wl.dtype)
        outs_like = [base[0]]
    if batched > 1:
        nbytes *= batched
    footprint = sum(t.numel() * t.element_size() for t in base + outs_like) * batched
    R = max(1, -(-512 * 1024 * 1024 // footprint))
    sets = []
    for r in range(R):
        ins = [t.clone() for t in base] if r else base
        sets.append((ins, [torch.empty_like(t) for t in outs_like]))
    stream = torch.cuda.current_stream(dev)
    if batched > 1:
        # K problems per buffer set, each with its own tensors
        bsets = []
        for r in range(R):
            bsets.append([dict(x=t[0].clone(), w_raw=t[1].clone(), lam=t[2].clone(), u=t[3].clone(),
                               out=torch.empty_like(base[0]), dirs=15, groups=wl.groups,
                               ch_per_weight=wl.cpw)
                          for t in [sets[r][0]] * batched])
        # descriptor arrays built once: a step is one call of the C ABI
        from linear_spatial_propagation_amd import _lib
        dtc = _lib.GSPN_BF16 if wl.dtype == "bf16" else _lib.GSPN_F32
        barrays = []
        for probs in bsets:
            arr = (_lib.Problem * batched)(*[
                _lib.Problem(pr["x"].data_ptr(), pr["w_raw"].data_ptr(), pr["lam"].data_ptr(),
                             pr["u"].data_ptr(), pr["out"].data_ptr(), B, C, H, W, 15, wl.groups, wl.cpw)
                for pr in probs])
            barrays.append(arr)
        batched_fn = _lib.load().gspn_scan_fwd_batched
        stream_handle = stream.cuda_stream

    # the plain forward and backward steps call the C ABI directly with
    # argument tuples built once, so host-side argument checks of the Python
    # binding stay out of the timed loop (the library validates every call)
    raw_fn, raw_args = None, []
    if batched == 1 and args.variant == "none":
        from linear_spatial_propagation_amd import _lib
        lib = _lib.load()
        dtc = _lib.GSPN_BF16 if wl.dtype == "bf16" else _lib.GSPN_F32
        raw_fn = lib.gspn_scan_bwd if bwd else lib.gspn_scan_fwd
        for ins, outs in sets:
            raw_args.append(tuple(t.data_ptr() for t in ins) + tuple(t.data_ptr() for t in outs) +
                            (B, C, H, W, 15, wl.groups, wl.cpw, dtc, stream.cuda_stream))

    def step_separate(i):
        for pr in bsets[i % R]:
            gspn.scan_fwd(pr["x"], pr["w_raw"], pr["lam"], pr["u"], dirs=15, groups=wl.groups,
                          ch_per_weight=wl.cpw, out=pr["out"])


    def step(i):
        ins, outs = sets[i % R]
        if raw_fn is not None:
            rc = raw_fn(*raw_args[i % R])
            if rc:
                _lib.check(rc)
        elif batched > 1:
            _lib.check(batched_fn(barrays[i % R], batched, dtc, stream_handle))
        elif bwd_variant:
            gspn.scan_bwd_dirs(*ins, dirs=15, groups=wl.groups, ch_per_weight=wl.cpw, out=outs)
        elif bwd:
            gspn.scan_bwd(*ins, dirs=15, groups=wl.groups, ch_per_weight=wl.cpw, out=outs)
        elif dirs_variant:
            gspn.scan_fwd_dirs(*ins, dirs=15, groups=wl.groups, ch_per_weight=wl.cpw, out=outs[0])
        else:
            gspn.scan_fwd(*ins, dirs=15, groups=wl.groups, ch_per_weight=wl.cpw, out=outs[0])

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)

    # timed region: K steps back to back, bracketed by two events on the
    # launch stream and device synchronisations (the throughput `value`)
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    w0 = time.perf_counter()
    t_all0.record(stream)
    for i in range(args.steps):
        step(i)
    t_all1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - w0
    elapsed = t_all0.elapsed_time(t_all1) * 1e-3

    # steady-state pass, independent of K: ROOF_WARM more untimed steps,
    # then ROOF_N steps back to back between one event pair (reported
    # beside the timed region; not the `value`)
    for i in range(ROOF_WARM):
        step(i)
    st0 = torch.cuda.Event(enable_timing=True)
    st1 = torch.cuda.Event(enable_timing=True)
    st0.record(stream)
    for i in range(ROOF_N):
        step(i)
    st1.record(stream)
    torch.cuda.synchronize(dev)
    steady = st0.elapsed_time(st1) * 1e-3 / ROOF_N

    # same-buffer ("hot") figure: the Infinity Cache may serve the inputs
    hot = None
    if not args.profile_run:
        hot_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(HOT_N)]
        for a, b in hot_ev:
            a.record(stream)
            step(0)
            b.record(stream)
        torch.cuda.synchronize(dev)
        hot = np.array([a.elapsed_time(b) for a, b in hot_ev]) * 1e-3

    separate_us = None
    if batched > 1:
        sep_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(min(args.steps, 100))]
        for i, (a, b) in enumerate(sep_ev):
            a.record(stream)
            step_separate(i)
            b.record(stream)
        torch.cuda.synchronize(dev)
        separate_us = float(np.median([a.elapsed_time(b) for a, b in sep_ev])) * 1e3

    if args.copy_calibration:
        src = torch.empty(COPY_CALIBRATION_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize(dev)

    # practical ceiling, for context: a plain device-to-device copy of
    # 2 x 512 MiB buffers (read + write bytes per second), median of 20
    copy_gbps = None
    if batched == 1 and not args.copy_calibration and not args.profile_run:   # the counter runs keep one known copy
        csrc = torch.empty(512 * 1024 * 1024, dtype=torch.uint8, device=dev)
        cdst = torch.empty_like(csrc)
        cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        cdst.copy_(csrc)
        for a, b in cev:
            a.record(stream)
            cdst.copy_(csrc)
            b.record(stream)
        torch.cuda.synchronize(dev)
        copy_gbps = round(2 * csrc.numel() / float(np.median([a.elapsed_time(b) for a, b in cev]) * 1e-3) / 1e9, 1)
        del csrc, cdst

    ms_per_step = elapsed / args.steps * 1e3
    value = nbytes * args.steps / elapsed / 1e9
    # roofline: algorithmic bytes over the average step of the timed region
    # (HIP events on the launch stream around the K back-to-back steps)
    achieved = nbytes / (elapsed / args.steps) / 1e9
    fwd_path = None if bwd or dirs_variant else gspn.select_path(B, C, H, W, groups=wl.groups, ch_per_weight=wl.cpw)
    # counter traffic exists for the single-kernel paths (fused forward and backward, slice)
    traffic_kernel = ("fused_bwd_kernel" if max(H, W) <= 64 else None) if bwd else (
        {1: "fused_scan_kernel", 3: "slice_scan_kernel"}.get(fwd_path))
    traffic = (load_traffic(args.pass_, traffic_kernel, args.config)
               if traffic_kernel and args.variant == "none" and batched == 1 else None)
    E = B * C * H * W
    out = {
        "metric": (METRIC_BWD_DIRS if bwd_variant else METRIC_BWD) if bwd else (METRIC_DIRS if dirs_variant else METRIC),
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{wl.dtype} I/O, f32 arithmetic",
        "data": "synthetic",
        "config": {
            "workload": f"{args.config}: B={B} C={C} H={H} W={W} groups={wl.groups} "
                        f"ch_per_weight={wl.cpw} dirs=TB|BT|LR|RL, {wl.dtype} I/O, fp32 arithmetic",
            "io_dtype": wl.dtype,
            "path": ("backward line kernels, per-direction lambda and u" if bwd_variant else
                     "fused backward" if max(H, W) <= 64 else "backward line kernels") if bwd else
                    "line kernels, per-direction lambda and u" if dirs_variant else
                    {1: "fused", 2: "general", 3: "slice"}[fwd_path],
            "algorithmic_bytes_per_step": nbytes,
            "buffer_sets": R,
            "seed": cfgd["seed"],
        },
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "elements_per_s": round(E * batched * args.steps / elapsed, 1),
        "step_us": round(elapsed / args.steps * 1e6, 3),
        "steady_state": {"steps": ROOF_N, "after_warmup": ROOF_WARM, "step_us": round(steady * 1e6, 3),
                         "gbps": round(nbytes / steady / 1e9, 2)},
        "hot_cache_gbps": round(nbytes / float(np.median(hot)) / 1e9, 2) if hot is not None else None,
        "device_copy_gbps": copy_gbps,
        "wall_s": round(wall, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic},
    }
    if dirs_variant:
        out["roofline"]["kernel"] = "gspn_scan_fwd_ex, all launches of one call"
    if batched > 1:
        out["metric"] = METRIC + f" ({batched} problems per batched launch)"
        out["config"]["batched_problems"] = batched
        out["config"]["path"] = "fused, batched"
        out["roofline"]["kernel"] = "fused_scan_batched_kernel"
        out["roofline"]["traffic"] = None
        out["separate_launches_us"] = round(separate_us, 3)
    if bwd:
        # 64 x 64 grids and smaller: one fused kernel per call
        out["roofline"]["kernel"] = ("gspn_scan_bwd_ex, all launches of one call" if bwd_variant else
                                     "fused_bwd_kernel" if max(H, W) <= 64
                                     else "gspn_scan_bwd, all launches of one call")
    if (not bwd and args.variant == "none" and batched == 1 and not args.profile_run and not args.copy_calibration
            and args.others):
        out["other_workloads"] = time_other_workloads(args.config, dev)
        out["backward"] = time_backward(cfgd, *bwd_inputs(cfgd, dev), dev)
    if not args.no_cpu and not args.profile_run and args.variant == "none" and batched == 1:
        out["cpu_baseline"] = cpu_baseline(args.config, backward=bwd)
    print(json.dumps(out), flush=True)


def time_other_workloads(skip, dev, warm=20, steps=200):
    """Forward time of every other workload of the suite, for context: inputs
    drawn on the device with the workloads' distributions (x ~ N(0, 1),
    lambda and u ~ U(0, 1), raw taps ~ N(0, 1)); 200 back-to-back calls on one
    buffer set after 20 untimed ones (the GPU's clocks settle over the first
    few dozen calls), HIP events on the launch stream.  Each entry also
    carries the workload's backward (`bwd`: one gspn_scan_bwd call per step,
    gy ~ N(0, 1), 50 calls after 10, outputs preallocated), whose algorithmic
    bytes are algorithmic_bytes_bwd's."""
    import torch
    import linear_spatial_propagation_amd as gspn
    from linear_spatial_propagation_amd import _lib
    from linear_spatial_propagation_amd.inputs import CONFIGS
    res = {}
    stream = torch.cuda.current_stream(dev)
    for name, c in CONFIGS.items():
        if name == skip or name == "tiny":
            continue
        B, C, H, W = c["B"], c["C"], c["H"], c["W"]
        dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
        g = torch.Generator(device=dev)
        g.manual_seed(c["seed"])
        nd = 4
        x = torch.randn((B, C, H, W), generator=g, device=dev, dtype=torch.float32).to(dt)
        w = torch.randn((nd, B, C // c["cpw"], 3, H, W), generator=g, device=dev, dtype=torch.float32).to(dt)
        lam = torch.rand((B, C, H, W), generator=g, device=dev, dtype=torch.float32).to(dt)
        if c["u_ones"]:
            u = torch.ones((B, C, H, W), device=dev, dtype=dt)
        else:
            u = torch.rand((B, C, H, W), generator=g, device=dev, dtype=torch.float32).to(dt)
        y = torch.empty_like(x)

        def step():
            gspn.scan_fwd(x, w, lam, u, dirs=15, groups=c["groups"], ch_per_weight=c["cpw"], out=y)
        for _ in range(warm):
            step()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize(dev)
        e0.record(stream)
        for _ in range(steps):
            step()
        e1.record(stream)
        torch.cuda.synchronize(dev)
        us = e0.elapsed_time(e1) * 1e3 / steps
        nbytes = algorithmic_bytes(B, C, H, W, 15, c["groups"], c["cpw"], c["dtype"])
        path = {1: "fused", 2: "general", 3: "slice"}[
            gspn.select_path(B, C, H, W, groups=c["groups"], ch_per_weight=c["cpw"],
                             dtype=_lib.GSPN_BF16 if c["dtype"] == "bf16" else _lib.GSPN_F32)]
        # the general path runs the line kernels where they hold the shape (the
        # backward's condition), else one scan per line
        if path == "general":
            path += " (line kernels)" if _lib.bwd_supported(B, C, H, W, groups=c["groups"], ch_per_weight=c["cpw"],
                                                             dtype=_lib.GSPN_BF16 if c["dtype"] == "bf16"
                                                             else _lib.GSPN_F32) == 0 else " (per line)"
        res[name] = {"path": path,
                     "us_per_step": round(us, 2), "gbps": round(nbytes / us / 1e3, 1),
                     "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}
        del y
        res[name]["bwd"] = time_backward(c, x, w, lam, u, g, dev)
        del x, w, lam, u
        torch.cuda.empty_cache()
    return res


def bwd_inputs(c, dev):
    """Device-drawn inputs of one workload for time_backward."""
    import torch
    B, C, H, W = c["B"], c["C"], c["H"], c["W"]
    dt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    g = torch.Generator(device=dev)
    g.manual_seed(c["seed"])
    x = torch.randn((B, C, H, W), generator=g, device=dev, dtype=torch.float32).to(dt)
    w = torch.randn((4, B, C // c["cpw"], 3, H, W), generator=g, device=dev, dtype=torch.float32).to(dt)
    lam = torch.rand((B, C, H, W), generator=g, device=dev, dtype=torch.float32).to(dt)
    u = (torch.ones((B, C, H, W), device=dev, dtype=dt) if c["u_ones"] else
         torch.rand((B, C, H, W), generator=g, device=dev, dtype=torch.float32).to(dt))
    return x, w, lam, u, g


def time_backward(c, x, w, lam, u, g, dev, warm=10, steps=50):
    """Backward time of one workload (see time_other_workloads)."""
    import torch
    import linear_spatial_propagation_amd as gspn
    B, C, H, W = c["B"], c["C"], c["H"], c["W"]
    gy = torch.randn(x.shape, generator=g, device=dev, dtype=torch.float32).to(x.dtype)
    outs = (torch.empty_like(x), torch.empty_like(w), torch.empty_like(x), torch.empty_like(x))
    stream = torch.cuda.current_stream(dev)

    def step():
        gspn.scan_bwd(x, w, lam, u, gy, dirs=15, groups=c["groups"], ch_per_weight=c["cpw"], out=outs)
    for _ in range(warm):
        step()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize(dev)
    us = e0.elapsed_time(e1) * 1e3 / steps
    nbytes = algorithmic_bytes_bwd(B, C, H, W, 15, c["groups"], c["cpw"], c["dtype"])
    del gy, outs
    return {"path": "fused" if max(H, W) <= 64 else "line kernels",
            "us_per_step": round(us, 2), "gbps": round(nbytes / us / 1e3, 1),
            "frac": round(nbytes / us / 1e3 / HBM_PEAK_GBPS, 4)}


if __name__ == "__main__":
    main()
