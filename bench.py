#!/usr/bin/env python3
"""Throughput of the bit-exact plane reductions on one MI355X.

One step = one batch through the whole path: the fused streaming kernel
(stage 1), the exact per-frame combine (stage 2), which writes the frames'
five sums (40 bytes each) straight into pinned host memory, and the host
conclusions (MSE, PSNR and the four moments) in libvqx.  Steps run on one
stream in groups of eight: each group ends with one completion event, and the
host concludes a group's batches while the GPU runs the next group (an
event record costs a few microseconds of command-processor time between
kernels, so there is one per group, not per step).  Stage 1 of every step is
timed with HIP events that its own dispatch stamps (hipExtLaunchKernel).  Inputs are resident in HBM before the
timed region; two copies of the batch alternate so that the 256 MB Infinity
Cache cannot serve a repeat.

Prints one JSON line.  ``roofline`` covers stage 1, timed live with HIP
events recorded around it on its own stream; ``cpu_baseline`` times the CPU
oracle (the CPU's sequential double arithmetic) on a bounded sample of the
same batch on this host's cores, and that leg also gates the result: the
timed batch must match the oracle (exact integers; bit-identical doubles
below 2^53 units; within the float_moment bound past it) or nothing is
reported.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5]
"""

from __future__ import annotations

import argparse
import ctypes
import gc
import hashlib
import json
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD's published peak
METRIC = "frames/s and HBM GB/s (fraction of peak) at 3840x2160 16-bit, bit-exact"
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCE = os.path.join(ROOT, "exact_reductions_amd", "csrc", "plane_stats.hip")


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    # Under sustained load the pass runs slower for its first tens of
    # milliseconds while the power manager settles (about 190 us per batch
    # at first, 156 us after ~55 ms); 300 warm-up steps (~55 ms) get past
    # that, and the timed steps measure steady streaming.
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--workload", type=int, default=5, help="workload number (5: 3840x2160 16-bit)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle leg (and with it the parity gate); for profiler runs")
    p.add_argument("--input-cache", default=None, metavar="DIR",
                   help="keep the generated batch as .npy files in DIR and reuse them")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="after the timed steps, run 3 elementwise kernels that each read and "
                        "write MIB MiB (the known-size kernel that scales the HBM counters)")
    return p.parse_args(argv)


def kernel_source_sha256() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^([A-Za-z0-9_]+):\s*(\S+)", line)
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("kernel_source_sha256") != kernel_source_sha256():
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class HipEvents:
    """Timing events from the HIP runtime torch and libvqx share."""

    def __init__(self, runtime: ctypes.CDLL):
        self.rt = runtime
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self) -> int:
        ev = ctypes.c_void_p()
        if self.rt.hipEventCreate(ctypes.byref(ev)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return ev.value

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        if self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def device_pointer(self, host_ptr: int) -> int:
        """Device address of pinned, mapped host memory (hipHostGetDevicePointer)."""
        self.rt.hipHostGetDevicePointer.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p,
                                                    ctypes.c_uint]
        out = ctypes.c_void_p()
        if self.rt.hipHostGetDevicePointer(ctypes.byref(out), ctypes.c_void_p(host_ptr), 0) != 0 or not out.value:
            raise RuntimeError("pinned host memory is not mapped for the device")
        return out.value

    def wait(self, stream: int, ev: int):
        self.rt.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
        if self.rt.hipStreamWaitEvent(ctypes.c_void_p(stream), ctypes.c_void_p(ev), 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def synchronize(self, ev: int):
        if self.rt.hipEventSynchronize(ctypes.c_void_p(ev)) != 0:
            raise RuntimeError("hipEventSynchronize failed")

    def record(self, ev: int, stream: int):
        if self.rt.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def destroy(self, ev: int):
        self.rt.hipEventDestroy(ctypes.c_void_p(ev))


def cpu_threads() -> int:
    """Host threads for the oracle: this process's CPU share, at most 16."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_and_gate(ref, dist, bpc, noise, moments, bytes_per_frame, concl):
    """Time the CPU oracle on a bounded sample and check the device's last
    batch, and the library's conclusion of it, against the oracle.  Returns
    (cpu_baseline dict, parity dict)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle

    nframes, h, w = ref.shape
    threads = cpu_threads()

    # parity of the timed batch: every frame, both oracles
    with ThreadPoolExecutor(threads) as ex:
        o2 = list(ex.map(lambda f: oracle.exact_frame_sums(ref[f], dist[f]), range(nframes)))
        o1 = list(ex.map(lambda f: oracle.seq_frame_sums(ref[f], dist[f], bpc), range(nframes)))
    failures = []
    past53 = 0
    for f in range(nframes):
        dev5 = [int(noise[f])] + [int(v) for v in moments[f]]
        fails = oracle.acceptance(dev5, o1[f], o2[f], w, h, bpc)
        want = oracle.conclude_from_ints(dev5, w, h, bpc)
        got = [concl[f, 0]] + list(concl[f, 2:])
        if got != list(want) or concl[f, 1] != oracle.psnr_db(want[0], bpc, 0.0):
            fails.append(("conclusion", f"{got} != {list(want)}"))
        if fails:
            failures.append((f, fails))
        past53 += sum(1 for v in o2[f] if int(v) >= oracle.TWO53)
    parity = {"frames": nframes, "failures": len(failures), "outputs_past_2^53": past53,
              "rule": "exact integers; doubles bit-identical below 2^53 units; bound past it"}
    if failures:
        parity["first_failure"] = str(failures[0])

    # timing: the oracle as it stands, one frame per task, on `threads` threads
    t = time.perf_counter()
    oracle.seq_frame_sums(ref[0], dist[0], bpc)
    one = max(time.perf_counter() - t, 1e-6)
    passes = max(1, min(50, int(12.0 / (one * nframes))))
    work = [f for _ in range(passes) for f in range(nframes)]
    t = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda f: oracle.seq_frame_sums(ref[f], dist[f], bpc), work))
    wall = time.perf_counter() - t
    fps = len(work) / wall
    base = {
        "value": round(fps, 3), "unit": "frames/s", "cores": threads, "kind": "oracle",
        "sample": f"{passes} passes over the {nframes} frames of the batch ({len(work)} frames of "
                  f"{w}x{h} at {bpc} bits), the C sequential-double oracle, one frame per task",
        "gbs": round(fps * bytes_per_frame / 1e9, 3),
        "single_thread_frames_per_s": round(1.0 / one, 3),
    }
    return base, parity


def load_or_generate(number, cache_dir):
    """The workload's batch, from ``cache_dir`` when it holds a copy whose
    digest matches the recipe's, else freshly generated (and stored there)."""
    import numpy as np

    import synth

    if not cache_dir:
        return synth.generate(number)
    os.makedirs(cache_dir, exist_ok=True)
    paths = [os.path.join(cache_dir, f"workload{number}_{p}.npy") for p in ("ref", "dist")]
    stamp = os.path.join(cache_dir, f"workload{number}.sha256")
    if all(os.path.exists(p) for p in paths + [stamp]):
        ref, dist = (np.load(p) for p in paths)
        with open(stamp) as f:
            if f.read().strip() == synth.sha256(ref, dist):
                return ref, dist
    ref, dist = synth.generate(number)
    for p, a in zip(paths, (ref, dist)):
        np.save(p, a)
    with open(stamp, "w") as f:
        f.write(synth.sha256(ref, dist))
    return ref, dist


def main(argv=None):
    args = parse_args(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the reduction shards by frames with no exchange, and no multi-GPU run is made here.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    from exact_reductions_amd import vqx

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    w, h, bpc, nframes = wl.w, wl.h, wl.bpc, wl.nframes

    t_gen = time.perf_counter()
    ref_np, dist_np = load_or_generate(args.workload, args.input_cache)
    t_gen = time.perf_counter() - t_gen

    # two resident copies of the batch, alternated step by step
    r0 = torch.from_numpy(ref_np).to(dev)
    d0 = torch.from_numpy(dist_np).to(dev)
    bufs = [(r0, d0), (r0.clone(), d0.clone())]
    # Sums land directly in pinned host memory that the GPU writes through
    # (zero-copy): stage 2 stores 40 bytes per frame there, and no copy
    # kernel runs.  `depth` groups of slots, so that the GPU always has
    # several groups queued while the host concludes the oldest one.
    group = 8
    depth = 4  # groups in flight: ~5 ms of queued work absorbs host hiccups
    nslots = depth * group
    sums = torch.zeros((nslots, 5 * nframes), dtype=torch.int64, pin_memory=True)
    noise = [sums[s, :nframes] for s in range(nslots)]
    moments = [sums[s, nframes:].view(nframes, 4) for s in range(nslots)]
    stream = torch.cuda.current_stream(dev)
    st = stream.cuda_stream
    ws_bytes = vqx.plane_stats_workspace_bytes(w, h, bpc, nframes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    hip = HipEvents(vqx.hip_runtime())
    L = vqx.lib()
    noise_dev = [hip.device_pointer(t.data_ptr()) for t in noise]
    moments_dev = [hip.device_pointer(t.data_ptr()) for t in moments]
    total = args.warmup + args.steps
    timed_every = 1
    ev_begin = {i: hip.create() for i in range(0, total, timed_every)}
    ev_end = {i: hip.create() for i in ev_begin}
    ev_done = [hip.create() for _ in range((total + group - 1) // group + 1)]
    torch.cuda.synchronize()

    # The host conclusion allocates nothing: libvqx concludes from the pinned
    # sums into preallocated arrays, and each step's sums are copied in place
    # into a preallocated history (to check afterwards that every step gave
    # the same sums).  Allocating numpy temporaries per batch stalled the
    # host for up to tens of milliseconds after the batch generation.
    sums_np = sums.numpy()
    concl = np.zeros((nslots, nframes, 6), dtype=np.float64)
    concl_ptr = [concl[s].ctypes.data for s in range(nslots)]
    noise_ptr = [noise[s].data_ptr() for s in range(nslots)]
    moments_ptr = [moments[s].data_ptr() for s in range(nslots)]
    history = np.zeros((total, 5 * nframes), dtype=np.int64)

    def enqueue(i):
        s = i % nslots
        r, d = bufs[i % 2]
        rc = L.vqx_plane_stats_batch_ws_timed(r.data_ptr(), d.data_ptr(), w, h, bpc, nframes,
                                              noise_dev[s], moments_dev[s], ws.data_ptr(), ws_bytes,
                                              st, ev_begin.get(i), ev_end.get(i))
        if rc != 0:
            raise vqx.VqxError(rc, "vqx_plane_stats_batch_ws_timed")

    def conclude(steps, done):
        hip.synchronize(done)
        for i in steps:
            s = i % nslots
            rc = L.vqx_conclude_batch(noise_ptr[s], moments_ptr[s], w, h, bpc, nframes, 0.0,
                                      concl_ptr[s])
            if rc != 0:
                raise vqx.VqxError(rc, "vqx_conclude_batch")
            history[i] = sums_np[s]

    def run(first, count):
        # step i uses slot i % nslots; a slot is reused only after the group
        # that last used it was concluded (at most `depth` groups in flight)
        groups = [list(range(a, min(a + group, first + count))) for a in range(first, first + count, group)]
        pending = []
        for steps in groups:
            if len(pending) == depth:
                conclude(*pending.pop(0))
            for i in steps:
                enqueue(i)
            done = ev_done[steps[0] // group]
            hip.record(done, st)
            pending.append((steps, done))
        while pending:
            conclude(*pending.pop(0))

    gc_was_enabled = gc.isenabled()
    gc.disable()
    try:
        if args.warmup > 0:
            run(0, args.warmup)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        run(args.warmup, args.steps)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
    finally:
        if gc_was_enabled:
            gc.enable()

    stage1_ms = [hip.elapsed_ms(ev_begin[i], ev_end[i]) for i in ev_begin if i >= args.warmup]
    for ev in list(ev_begin.values()) + list(ev_end.values()) + ev_done:
        hip.destroy(ev)

    # every step must have produced the same sums
    if not np.all(history == history[total - 1]):
        bad = int(np.nonzero(np.any(history != history[total - 1], axis=1))[0][0])
        print(f"step {bad} differs from the last step", file=sys.stderr)
        return 1
    last_noise = history[total - 1, :nframes]
    last_moments = history[total - 1, nframes:].reshape(nframes, 4)
    # the library's conclusion of the last step, from the same sums
    last_concl = concl[(total - 1) % nslots].copy()

    if args.calibrate_copy:
        # a kernel that reads exactly n bytes and writes exactly n bytes
        n = args.calibrate_copy * (1 << 20)
        src = torch.ones(n // 4, dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.bitwise_not(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    bytes_per_frame = wl.bytes_per_frame
    bytes_per_launch = bytes_per_frame * nframes
    mean_stage1 = statistics.fmean(stage1_ms)
    achieved = bytes_per_launch / (mean_stage1 * 1e-3) / 1e9
    kernel = "stage1_u8" if bpc == 8 else "stage1_u16"
    wname = f"{w}x{h}x{nframes}_{bpc}bit"
    traffic = stored_traffic(kernel, wname)

    out = {
        "metric": METRIC,
        "value": round(args.steps * nframes / elapsed, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 squares, u64 sums",
        "data": "synthetic",
        "config": {
            "workload": f"{w}x{h} {bpc}-bit luma pair, {nframes} frames, "
                        f"{'uint8' if bpc == 8 else 'uint16'} ({wl.recipe})",
            "w": w, "h": h, "bpc": bpc, "nframes": nframes,
            "bytes_per_step": bytes_per_launch,
            "hbm_gbs_whole_step": round(bytes_per_launch * args.steps / elapsed / 1e9, 1),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "kernel_us_mean": round(mean_stage1 * 1e3, 2),
            "kernel_us_median": round(statistics.median(stage1_ms) * 1e3, 2),
            "algorithmic_bytes_per_launch": bytes_per_launch,
        },
        "generation_s": round(t_gen, 1),
    }

    if not args.no_cpu_baseline:
        base, parity = cpu_baseline_and_gate(ref_np, dist_np, bpc, last_noise, last_moments,
                                             bytes_per_frame, last_concl)
        out["cpu_baseline"] = base
        out["parity"] = parity
        if parity["failures"]:
            print(json.dumps({"error": "timed batch does not match the oracle", "parity": parity}),
                  file=sys.stderr)
            return 1
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
