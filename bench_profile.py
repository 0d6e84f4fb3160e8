#!/usr/bin/env python3
"""rocprofv3 passes over bench.py and short text summaries of them.

Runs, each as a child process under its own time limit:

1. ``rocprofv3 --kernel-trace --stats`` over a bench run: per-kernel call
   counts and durations (the stage-1 average must agree with the HIP-event
   figure bench.py reports);
2. ``rocprofv3 --pmc FETCH_SIZE`` and 3. ``rocprofv3 --pmc WRITE_SIZE``, one
   counter per run, over a short bench run that also runs three elementwise
   kernels that each read and write a known 1 GiB (a plain streaming copy
   through the shader cores); that kernel's counter reading scales the
   stage-1 reading into HBM bytes.

With ``--valu``, one counter pass instead: instructions per dispatch and
how busy the SIMDs were (``..._valu.txt``).  With ``--driver-cmd``, only 1.,
over the default command
``bench.py --gpus 1 --steps 20 --warmup 5`` as it is run for the record:
``<kernel>_<w>x<h>x<frames>_driver_cmd_kernel_trace.txt``.

Writes ``<kernel>_<w>x<h>x<frames>_kernel_trace.txt`` and
``..._hbm_traffic.txt`` into ``--out``.  With ``--mode cpu-order`` the
kernel is the whole CPU-order step (``cpu_order_step``): the trace lists
each of its kernels, and the traffic sums their counters per step.  This
script never touches the GPU itself.

    python bench_profile.py --workload 5 [--mode cpu-order] --out <summaries> --work <work>

The raw rocprofv3 output goes under ``--work``; the summaries record their
commands with that directory written as ``<work>``.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import shlex
import statistics
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
COPY_MIB = 1024
WARMUP = 300


def sh(cmd, timeout, log):
    print(f"[bench_profile] {' '.join(shlex.quote(c) for c in cmd)}", flush=True)
    with open(log, "w") as f:
        r = subprocess.run(["timeout", "-s", "KILL", str(timeout)] + cmd, stdout=f, stderr=subprocess.STDOUT)
    print(f"[bench_profile] exit {r.returncode}", flush=True)
    return r.returncode


def find(pattern_dir, suffix):
    hits = sorted(glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {pattern_dir}")
    return hits[-1]


def shown(cmd, args) -> str:
    """A command as the summaries record it: repository paths relative, the
    raw-output directory as <work>."""
    text = " ".join(shlex.quote(c) for c in cmd)
    work = os.path.abspath(args.work)
    text = text.replace(work, "<work>")
    rel = os.path.relpath(work, ROOT)
    if not rel.startswith(".."):
        text = text.replace(rel, "<work>")
    return text.replace(ROOT + "/", "")


def rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def short(name: str) -> str:
    for k in ("stage1_u16_mapped", "mapped_combine", "gather_view", "stage1_u16", "stage1_u8", "stage2_combine",
              "bitwise_not", "fsum_tile_totals", "fsum_plan", "fsum_tile_maps", "fsum_walk",
              "cpu_order_maps", "cpu_order_walk", "views_stage1", "views_combine",
              "view_stage1", "view_combine", "read_probe"):
        if k in name:
            return k
    return name.split("(")[0][-60:]


def _union(intervals):
    out = []
    for b, e in sorted(intervals):
        if out and b <= out[-1][1]:
            out[-1][1] = max(out[-1][1], e)
        else:
            out.append([b, e])
    return out


def _overlap(a, b):
    """Total length of the intersection of two unions of intervals."""
    i = j = 0
    total = 0
    while i < len(a) and j < len(b):
        lo = max(a[i][0], b[j][0])
        hi = min(a[i][1], b[j][1])
        if hi > lo:
            total += hi - lo
        if a[i][1] < b[j][1]:
            i += 1
        else:
            j += 1
    return total


def profile_host(args, wl, wname, bench, src_sha):
    """Kernel and memory-copy trace of the host-fed mode: the uploads, the
    kernels, and how much of the kernels' time runs while an upload is in
    flight (the overlap the two streams are for)."""
    rc = sh(bench + ["--steps", "1", "--warmup", "0", "--no-cpu-baseline"], 600,
            os.path.join(args.work, "prime.log"))
    if rc != 0:
        return rc
    tdir = os.path.join(args.work, "trace")
    steps = 20
    cmd = ["rocprofv3", "--kernel-trace", "--memory-copy-trace", "--stats", "--output-format", "csv", "-d", tdir,
           "-o", "trace", "--"] + bench + ["--steps", str(steps), "--warmup", "3"]
    rc = sh(cmd, 300, os.path.join(args.work, "trace.log"))
    if rc != 0:
        return rc
    with open(os.path.join(args.work, "trace.log")) as f:
        bench_line = [ln for ln in f.read().splitlines() if ln.startswith("{")]
    kernels = rows(find(tdir, "kernel_trace.csv"))
    copies = rows(find(tdir, "memory_copy_trace.csv"))
    kint = _union([(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in kernels
                   if short(r["Kernel_Name"]) in ("stage1_u16", "stage1_u8", "stage2_combine")])
    h2d = [r for r in copies if "HOST_TO_DEVICE" in (r.get("Direction", "") + r.get("Kind", "")).upper()
           or "H2D" in (r.get("Direction", "") + r.get("Kind", "")).upper()]
    cint = _union([(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in h2d])
    k_time = sum(e - b for b, e in kint)
    c_time = sum(e - b for b, e in cint)
    both = _overlap(kint, cint)
    lines = [
        f"# rocprofv3 kernel and memory-copy trace: host-fed step, {wl.name} ({wname}), "
        f"{args.frames_per_upload} frames per upload",
        f"command: cd <repo> && {shown(cmd, args)}",
        f"date_utc: {time.strftime('%Y-%m-%dT%H:%M:%SZ', time.gmtime())}",
        f"kernel_source_sha256: {src_sha}",
        "",
        f"{'kernel':<18} {'calls':>6} {'avg_us':>10} {'total_us':>12}",
    ]
    for r in rows(find(tdir, "kernel_stats.csv")):
        lines.append(f"{short(r.get('Name', '?')):<18} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['TotalDurationNs']) / 1e3:>12.1f}")
    lines += [
        "",
        f"host_to_device_copies: {len(h2d)} (all copies in the trace: {len(copies)}; kinds: "
        f"{sorted({(r.get('Kind', ''), r.get('Direction', '')) for r in copies})})",
        f"copy_busy_ms: {c_time / 1e6:.2f}",
        f"kernel_busy_ms: {k_time / 1e6:.2f}",
        f"kernel_time_under_a_copy_ms: {both / 1e6:.2f}",
        f"kernel_time_hidden_fraction: {both / k_time:.4f}" if k_time else "kernel_time_hidden_fraction: n/a",
        "(the trace also holds the bench's plain-upload timing, copies with no kernel beside them)",
    ]
    if bench_line:
        lines += ["", "bench line of the same run:", bench_line[-1]]
    with open(os.path.join(args.out, f"host_step_{wname}_trace.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)
    return 0


def kernel_trace(args, trace_cmd, steps, warmup, title, outname, step_kernels, src_sha, alg):
    """Run ``trace_cmd`` (rocprofv3 --kernel-trace --stats over a bench run
    of ``warmup`` + ``steps`` steps) and write its summary as ``outname``.
    Returns (exit status, dispatches per step of each of the step's kernels)."""
    tdir = trace_cmd[trace_cmd.index("-d") + 1]
    rc = sh(trace_cmd, 300, os.path.join(args.work, "trace.log"))
    if rc != 0:
        return rc, {}
    stats = rows(find(tdir, "kernel_stats.csv"))
    with open(os.path.join(args.work, "trace.log")) as f:
        bench_line = [ln for ln in f.read().splitlines() if ln.startswith("{")]
    lines = [
        f"# rocprofv3 kernel trace: {title}",
        f"command: cd <repo> && {shown(trace_cmd, args)}",
        f"date_utc: {time.strftime('%Y-%m-%dT%H:%M:%SZ', time.gmtime())}",
        f"kernel_source_sha256: {src_sha}",
        "",
        f"{'kernel':<18} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_us':>12}",
    ]
    for r in stats:
        name = short(r.get("Name", r.get("KernelName", "?")))
        lines.append(f"{name:<18} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.2f} "
                     f"{float(r['MinNs']) / 1e3:>10.2f} {float(r['MaxNs']) / 1e3:>10.2f} "
                     f"{float(r['TotalDurationNs']) / 1e3:>12.1f}")
    # each kernel's dispatches in launch order, from the trace; the bench
    # times the dispatches after its warm-up ones
    trace = rows(find(tdir, "kernel_trace.csv"))
    timed_avg = {}
    per_step = {}
    for kname in step_kernels:
        disp = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in trace
                      if short(r["Kernel_Name"]) == kname)
        k = max(1, round(len(disp) / (warmup + steps)))  # dispatches of this kernel per step
        timed = [(e - b) / 1e3 for b, e in disp[k * warmup:]]
        if timed:
            timed_avg[kname] = statistics.fmean(timed)
            per_step[kname] = k
            lines += ["", f"{kname}: dispatches {len(disp)}, {k} per step (the first {k * warmup} are the "
                          "bench's warm-up)",
                      f"{kname}_avg_us_timed_dispatches: {statistics.fmean(timed):.2f}",
                      f"{kname}_median_us_timed_dispatches: {statistics.median(timed):.2f}",
                      f"{kname}_min_us_timed_dispatches: {min(timed):.2f}",
                      f"{kname}_max_us_timed_dispatches: {max(timed):.2f}"]
    if len(timed_avg) == len(step_kernels):
        step_us = sum(timed_avg[k] * per_step[k] for k in step_kernels)
        how = "  (sum of the step's kernels)" if len(step_kernels) > 1 else ""
        if len(step_kernels) > 1:
            # kernels of a step may run at once on two streams: the step is
            # the span from its first kernel's start to its last one's end
            disp = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), short(r["Kernel_Name"]))
                          for r in trace if short(r["Kernel_Name"]) in step_kernels)
            spans, cur = [], None
            for b, e, kname in disp:
                if kname == step_kernels[0]:
                    if cur:
                        spans.append(cur[1] - cur[0])
                    cur = [b, e]
                elif cur:
                    cur[1] = max(cur[1], e)
            if cur:
                spans.append(cur[1] - cur[0])
            spans = [x / 1e3 for x in spans[warmup:]]
            if spans:
                step_us = statistics.fmean(spans)
                how = "  (per step, the first kernel's start to the last kernel's end)"
                lines += ["", f"step_span_us_timed_steps: mean {step_us:.2f}, median "
                              f"{statistics.median(spans):.2f}, min {min(spans):.2f}, max {max(spans):.2f} "
                              f"over {len(spans)} steps"]
        gbs = alg / (step_us * 1e-6) / 1e9
        lines += ["", f"kernel_avg_us: {step_us:.2f}" + how,
                  f"kernel_algorithmic_bytes_per_launch: {alg}",
                  f"kernel_achieved_GBps: {gbs:.1f}", f"kernel_frac_of_8000_GBps: {gbs / 8000:.4f}"]
    if bench_line:
        lines += ["", "bench line of the same run:", bench_line[-1]]
    with open(os.path.join(args.out, outname), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)
    return 0, per_step


VALU_COUNTERS = ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS", "SQ_WAVES",
                 "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")


def profile_valu(args, wl, wname, kernel, step_kernels, bench, src_sha):
    """One counter pass (seven counters, within one pass's limits) over a
    short bench run: vector and scalar instructions, loads and LDS
    instructions per dispatch, and how busy the SIMDs were."""
    cdir = os.path.join(args.work, "valu")
    cmd = ["rocprofv3", "--pmc", *VALU_COUNTERS, "--output-format", "csv", "-d", cdir, "-o", "p", "--"] + bench + [
        "--steps", "5", "--warmup", "1"]
    rc = sh(cmd, 120, os.path.join(args.work, "valu.log"))
    if rc != 0:
        return rc
    per = {}
    for r in rows(find(cdir, "counter_collection.csv")):
        per.setdefault((short(r["Kernel_Name"]), r["Counter_Name"]), []).append(float(r["Counter_Value"]))
    lines = [
        f"# VALU counters of {kernel}, {wl.name} ({wname})",
        f"command: cd <repo> && {shown(cmd, args)}",
        f"date_utc: {time.strftime('%Y-%m-%dT%H:%M:%SZ', time.gmtime())}",
        f"kernel_source_sha256: {src_sha}",
        "",
        "per-dispatch means over the run's dispatches (counters summed over the device, as rocprofv3 reports them):",
    ]
    names = sorted({k for k, _ in per})
    for name in names:
        for c in VALU_COUNTERS:
            v = per.get((name, c))
            if v:
                lines.append(f"  {name:<18} {c:<17} n={len(v):>2} mean={statistics.fmean(v):.6g}")
    lines += ["", "VALU busy = SQ_INSTS_VALU x 4 cycles (a wave64 instruction on a 16-lane SIMD; plain fp32 and",
              "            32-bit integer instructions issue faster on gfx950, so this is an upper bound) /",
              "            (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs):"]
    for name in names:
        v, g = per.get((name, "SQ_INSTS_VALU")), per.get((name, "GRBM_GUI_ACTIVE"))
        if v and g:
            lines.append(f"  {name:<18} {statistics.fmean(v) * 4 / (statistics.fmean(g) / 8 * 1024):.3f}")
    pixels = wl.w * wl.h * wl.nframes
    for name in step_kernels:
        v = per.get((name, "SQ_INSTS_VALU"))
        if v:
            lines.append(f"  {name}: {statistics.fmean(v) * 64 / pixels:.2f} VALU lane instructions per pixel pair "
                         "(all of the kernel's instructions over the batch's pixel pairs)")
    with open(os.path.join(args.out, f"{kernel}_{wname}_valu.txt"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines), flush=True)
    return 0


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--workload", type=int, default=None)
    p.add_argument("--out", default=os.path.join(ROOT, "_prof", "summaries"))
    p.add_argument("--work", default=os.path.join(ROOT, "_prof", "rocprof"))
    p.add_argument("--cache", default="/tmp/vqx_inputs")
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--frames-per-upload", type=int, default=4)
    p.add_argument("--mode", choices=("exact", "cpu-order", "psnr-int", "yuv420", "host", "hvs-sum"),
                   default="exact")
    p.add_argument("--planes", type=int, default=32, help="hvs-sum mode: term buffers per step")
    p.add_argument("--pitch", type=int, default=0, help="as bench.py --pitch")
    p.add_argument("--x0", type=int, default=0, help="as bench.py --x0")
    p.add_argument("--valu", action="store_true", help="the VALU counter pass only")
    p.add_argument("--driver-cmd", action="store_true",
                   help="kernel trace only, over the plain default run: bench.py --gpus 1 --steps 20 --warmup 5")
    args = p.parse_args(argv)
    cpu_order = args.mode == "cpu-order"
    views = args.mode in ("psnr-int", "yuv420")
    if args.workload is None:
        args.workload = 2 if args.mode == "yuv420" else 5

    sys.path.insert(0, ROOT)
    import bench as bench_mod
    import synth
    wl = synth.WORKLOADS[args.workload]
    if args.pitch == wl.w and not args.x0:
        args.pitch = 0
    x0 = args.x0 if args.pitch else 0
    # the same plan as the bench's own (its summaries are looked up by name and sources)
    kernel, step_kernels, sources = bench_mod.step_plan(args.mode, wl, args.pitch, x0)
    wname = (f"{wl.w}x{wl.h}x{wl.nframes}_{wl.bpc}bit" + ("_yuv420" if args.mode == "yuv420" else "")
             + (f"_pitch{args.pitch}" if args.pitch else "") + (f"_x{x0}" if x0 else ""))
    os.makedirs(args.out, exist_ok=True)
    os.makedirs(args.work, exist_ok=True)
    bench = ["python3", os.path.join(ROOT, "bench.py"), "--workload", str(args.workload),
             "--no-cpu-baseline", "--input-cache", args.cache, "--mode", args.mode]
    if args.mode == "host":
        bench += ["--frames-per-upload", str(args.frames_per_upload)]
    if args.pitch:
        bench += ["--pitch", str(args.pitch)]
    if x0:
        bench += ["--x0", str(x0)]
    h = hashlib.sha256()
    for path in sources:
        with open(path, "rb") as f:
            h.update(f.read())
    src_sha = h.hexdigest()
    alg = wl.bytes_per_frame * wl.nframes
    if args.mode == "yuv420":
        frame = wl.w * wl.h + 2 * (-(-wl.w // 2)) * (-(-wl.h // 2))
        alg = 2 * frame * wl.bytes_per_sample * wl.nframes
    if cpu_order:
        ref, dist = synth.generate(args.workload)
        alg += bench_mod.past53_bytes(ref, dist, wl.bpc)
        del ref, dist
    if args.mode == "hvs-sum":
        bw, bh = synth.HVS_4K_BLOCKS
        wname = f"3840x2160x{args.planes}_hvs"
        alg = 4 * bw * bh * 64 * args.planes  # one read of the terms
        bench += ["--planes", str(args.planes)]
        wl = synth.Workload(0, f"{args.planes} psnr_hvs-like term buffers of a 3840x2160 plane", 3840, 2160,
                            args.planes, 16, "psnr_hvs-like terms")

    if args.mode == "host":
        return profile_host(args, wl, wname, bench, src_sha)

    if args.valu:
        return profile_valu(args, wl, wname, kernel, step_kernels, bench, src_sha)

    if args.driver_cmd:
        # the default bench command as it is run for the record (default
        # workload and mode, cpu_baseline leg included), traced as it is
        drv = ["python3", os.path.join(ROOT, "bench.py"), "--gpus", "1", "--steps", "20", "--warmup", "5"]
        trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                     os.path.join(args.work, "trace"), "-o", "trace", "--"] + drv
        return kernel_trace(args, trace_cmd, 20, 5, f"{kernel}, {wl.name} ({wname}), the default bench command",
                            f"{kernel}_{wname}_driver_cmd_kernel_trace.txt", step_kernels, src_sha, alg)[0]

    # 0. make the input cache outside the profiler
    rc = sh(bench + ["--steps", "1", "--warmup", "0"], 600, os.path.join(args.work, "prime.log"))
    if rc != 0:
        return rc

    # 1. kernel trace + stats
    trace_cmd = ["rocprofv3", "--kernel-trace", "--stats", "--output-format", "csv", "-d",
                 os.path.join(args.work, "trace"), "-o", "trace", "--"] + bench + ["--steps", str(args.steps),
                                                                                  "--warmup", str(WARMUP)]
    rc, per_step = kernel_trace(args, trace_cmd, args.steps, WARMUP, f"{kernel}, {wl.name} ({wname})",
                                f"{kernel}_{wname}_kernel_trace.txt", step_kernels, src_sha, alg)
    if rc != 0:
        return rc

    # 2./3. one counter per pass
    readings = {}
    cmds = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        cdir = os.path.join(args.work, counter.lower())
        cmd = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", cdir, "-o", counter.lower(),
               "--"] + bench + ["--steps", "5", "--warmup", "1", "--calibrate-copy", str(COPY_MIB)]
        cmds[counter] = cmd
        rc = sh(cmd, 240, os.path.join(args.work, f"{counter.lower()}.log"))
        if rc != 0:
            return rc
        per_kernel = {}
        for r in rows(find(cdir, "counter_collection.csv")):
            if r.get("Counter_Name") != counter:
                continue
            per_kernel.setdefault(short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        readings[counter] = per_kernel

    copy_bytes = COPY_MIB * (1 << 20)
    out = [
        f"# HBM traffic of {kernel}, {wl.name} ({wname}), from rocprofv3 counters"
        + (f" (summed over {', '.join(step_kernels)} per step)" if len(step_kernels) > 1 else ""),
        f"command_fetch: cd <repo> && {shown(cmds['FETCH_SIZE'], args)}",
        f"command_write: cd <repo> && {shown(cmds['WRITE_SIZE'], args)}",
        f"date_utc: {time.strftime('%Y-%m-%dT%H:%M:%SZ', time.gmtime())}",
        f"kernel_source_sha256: {src_sha}",
        f"copy_kernel_bytes_read_and_written: {copy_bytes}",
        "",
        "per-dispatch means (KiB as the counter reports them):",
    ]
    for counter, per_kernel in readings.items():
        for name, vals in sorted(per_kernel.items()):
            out.append(f"  {counter:<10} {name:<48} n={len(vals):<3} mean={statistics.fmean(vals):.1f}")
    # the known-size kernel: torch's bitwise_not over 1 GiB (its last three
    # dispatches; earlier bitwise_not dispatches, if any, are not ours)
    def copy_reading(per_kernel):
        vals = per_kernel.get("bitwise_not")
        return statistics.fmean(vals[-3:]) if vals else None
    fetch_copy = copy_reading(readings["FETCH_SIZE"])
    write_copy = copy_reading(readings["WRITE_SIZE"])
    # per step: the mean per dispatch of each of the step's kernels, summed
    have = all(readings[c].get(k) for c in ("FETCH_SIZE", "WRITE_SIZE") for k in step_kernels)
    if fetch_copy and write_copy and have:
        f_scale = copy_bytes / fetch_copy
        w_scale = copy_bytes / write_copy
        ps = {k: per_step.get(k, 1) for k in step_kernels}
        fetch_b = sum(statistics.fmean(readings["FETCH_SIZE"][k]) * ps[k] for k in step_kernels) * f_scale
        write_b = sum(statistics.fmean(readings["WRITE_SIZE"][k]) * ps[k] for k in step_kernels) * w_scale
        out += [
            "",
            f"fetch_scale_bytes_per_unit: {f_scale:.4f}",
            f"write_scale_bytes_per_unit: {w_scale:.4f}",
            f"kernel_fetch_bytes_per_launch: {fetch_b:.0f}",
            f"kernel_write_bytes_per_launch: {write_b:.0f}",
            f"hbm_bytes_per_launch: {fetch_b + write_b:.0f}",
            f"algorithmic_bytes_per_launch: {alg}",
            f"traffic_over_algorithmic: {(fetch_b + write_b) / alg:.4f}",
        ]
        if len(step_kernels) > 1:
            for k in step_kernels:
                out.append(f"  {k}: fetch {statistics.fmean(readings['FETCH_SIZE'][k]) * f_scale:.0f} "
                           f"write {statistics.fmean(readings['WRITE_SIZE'][k]) * w_scale:.0f} bytes per dispatch")
    with open(os.path.join(args.out, f"{kernel}_{wname}_hbm_traffic.txt"), "w") as f:
        f.write("\n".join(out) + "\n")
    print("\n".join(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
