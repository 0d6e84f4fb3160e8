#!/usr/bin/env python3
"""Throughput of the bit-exact plane reductions on one MI355X.

One step = one batch through the whole path: the fused streaming kernel
(stage 1), the exact per-frame combine (stage 2), the 40-byte-per-frame copy
of the sums to pinned host memory, and the host conclusions (MSE, PSNR and
the four moments) in libvqx.  Steps are pipelined: the host concludes batch
i-1 while the GPU works on batch i.  Inputs are resident in HBM before the
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
    # The first ~10 ms of sustained load run at reduced clocks while the
    # power manager settles; 100 warm-up steps (~18 ms) get past that, and
    # the timed steps measure steady streaming.
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=100)
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


def cpu_baseline_and_gate(ref, dist, bpc, noise, moments, bytes_per_frame):
    """Time the CPU oracle on a bounded sample and check the device's last
    batch against it.  Returns (cpu_baseline dict, parity dict)."""
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
    # kernel runs.  Two slots, so that batch i+1 can be queued while the host
    # concludes batch i.
    sums = torch.zeros((2, 5 * nframes), dtype=torch.int64, pin_memory=True)
    noise = [sums[s, :nframes] for s in range(2)]
    moments = [sums[s, nframes:].view(nframes, 4) for s in range(2)]
    ws_bytes = vqx.plane_stats_workspace_bytes(w, h, bpc, nframes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    hip = HipEvents(vqx.hip_runtime())
    L = vqx.lib()
    noise_dev = [hip.device_pointer(t.data_ptr()) for t in noise]
    moments_dev = [hip.device_pointer(t.data_ptr()) for t in moments]
    total = args.warmup + args.steps
    ev_begin = [hip.create() for _ in range(total + 1)]
    ev_end = [hip.create() for _ in range(total)]
    torch.cuda.synchronize()

    results = {}

    def enqueue(i):
        # the begin event of step i also marks the end of step i-1 (same stream)
        r, d = bufs[i % 2]
        rc = L.vqx_plane_stats_batch_ws_timed(r.data_ptr(), d.data_ptr(), w, h, bpc, nframes,
                                              noise_dev[i % 2], moments_dev[i % 2], ws.data_ptr(),
                                              ws_bytes, stream.cuda_stream, ev_begin[i], ev_end[i])
        if rc != 0:
            raise vqx.VqxError(rc, "vqx_plane_stats_batch_ws_timed")

    def conclude(i):
        # wait for step i (the next begin event, or a final marker), then conclude it
        if hip.rt.hipEventSynchronize(ctypes.c_void_p(ev_begin[i + 1])) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        s = i % 2
        results[i] = (vqx.conclude_batch(noise[s].numpy(), moments[s].numpy(), w, h, bpc),
                      noise[s].numpy().copy(), moments[s].numpy().copy())

    def run(first, count):
        for i in range(first, first + count):
            enqueue(i)
            if i > first:
                conclude(i - 1)
        last = first + count - 1
        hip.record(ev_begin[last + 1], stream.cuda_stream)
        conclude(last)

    if args.warmup > 0:
        run(0, args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run(args.warmup, args.steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    stage1_ms = [hip.elapsed_ms(ev_begin[i], ev_end[i]) for i in range(args.warmup, total)]
    for ev in ev_begin + ev_end:
        hip.destroy(ev)

    # every timed step must have produced the same sums
    last = results[total - 1]
    for i in range(args.warmup, total):
        if not (np.array_equal(results[i][1], last[1]) and np.array_equal(results[i][2], last[2])):
            print(f"step {i} differs from the last step", file=sys.stderr)
            return 1

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
    wname = f"{w}x{h}x{nframes}"
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
            "stage1_us_mean": round(mean_stage1 * 1e3, 2),
            "stage1_us_median": round(statistics.median(stage1_ms) * 1e3, 2),
            "algorithmic_bytes_per_launch": bytes_per_launch,
        },
        "generation_s": round(t_gen, 1),
    }

    if not args.no_cpu_baseline:
        base, parity = cpu_baseline_and_gate(ref_np, dist_np, bpc, last[1], last[2], bytes_per_frame)
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
