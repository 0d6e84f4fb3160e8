#!/usr/bin/env python3
"""Throughput of the bit-exact plane reductions on one MI355X.

One step = one batch through the whole path: the fused streaming kernel
(stage 1), the exact per-frame combine (stage 2), which writes the frames'
five sums (40 bytes each) straight into pinned host memory, and the host
conclusions (MSE, PSNR and the four moments) in libvqx.  Steps run on one
stream by default; ``--streams N`` alternates them over N streams (step i on
stream i % N, each with its own workspace), as a pipeline of batches would,
and then consecutive steps overlap and a kernel's timed duration includes the
overlap.
Steps go in groups of eight: a group starts on every stream after one start
event, ends when every stream has finished its steps of the group, and ends
with one completion event; the host concludes a group's batches while the GPU
runs the next group (an event record costs a few microseconds of
command-processor time between kernels, so there is one per group, not per
step).  Stage 1 of every step is
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

``read_ceiling`` (this mode only) times the library's read probe, which
reads the same batch with stage 1's grid, chunks and loads but does no
arithmetic: the practical read ceiling of stage 1's access pattern, beside
which stage 1's own time is put.

``--mode cpu-order`` measures the other entry point instead: each step also
reproduces the CPU's own rounding past 2^53 (vqx_plane_stats_batch_cpu_order_ws:
stage 1, the prefix scan, which also writes the exact sums, the maps pass
over the chunks past 2^53 inside which adds can round, the chunk and block
maps, the walk), and the host concludes those sums.
Its roofline is the whole step against the bytes it must read (both planes
once, and those chunks again), timed with HIP events around each group of
steps; the gate is bit-identity with the oracle's sequential doubles on
every frame.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--mode exact|cpu-order]
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
METRIC_CPU_ORDER = ("frames/s with the CPU's own rounding past 2^53 (sums bit-identical to the "
                    "sequential doubles) at 3840x2160 16-bit")
METRIC_PSNR_INT = "frames/s of the integer psnr twin (exact uint64 sum of (ref - dist)^2 per frame)"
METRIC_YUV420 = ("frames/s of the integer psnr twin on all three planes of planar 4:2:0 frames "
                 "(Y, U, V through plane views)")
METRIC_HOST = ("frames/s of the exact sums of a batch in pinned host memory, PCIe upload included "
               "(3840x2160 16-bit)")
METRIC_HVS_SUM = ("frames/s of the psnr_hvs running float sum of 3840x2160 luma planes (10 802 176 terms "
                  "each, the float bit-identical to the CPU's sequential sum)")
PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction, the published link rate
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "exact_reductions_amd", "csrc")
STAGE1_SOURCES = [os.path.join(CSRC, f) for f in ("plane_stats.hip", "reduce.h")]
CPU_ORDER_SOURCES = STAGE1_SOURCES + [os.path.join(CSRC, "cpu_order.hip")]
VIEW_SOURCES = [os.path.join(CSRC, f) for f in ("plane_views.hip", "reduce.h")]
HOST_SOURCES = STAGE1_SOURCES + [os.path.join(CSRC, "host_stream.hip")]
MAPPED_SOURCES = [os.path.join(CSRC, f) for f in ("stage1_mapped.hip", "reduce.h")]
FLOAT_SUM_SOURCES = [os.path.join(CSRC, "float_sum.hip")]
FLOAT_SUM_KERNELS = ("fsum_tile_totals", "fsum_plan", "fsum_tile_maps", "fsum_walk")
CPU_ORDER_KERNELS = ("stage1_u16", "cpu_order_maps", "cpu_order_walk")


def step_plan(mode: str, wl, pitch: int = 0, x0: int = 0):
    """(kernel, step kernels, sources) of a bench mode: the name of the timed
    step's dominant kernel (or of the whole step), the kernels one step runs
    as rocprofv3 names them, and the sources they are built from.  Planes
    with a pitch (rows of ``pitch`` samples, the frame ``x0`` samples into
    each) go through the view entry points, which read rows of whole 16-byte
    vectors of two-byte samples in place with the contiguous chunks
    ("mapped": aligned vectors for the exact sums, vectors at any offsets
    within 16 bytes for the CPU-order form) and gather or tile other
    layouts."""
    vectors = bool(pitch) and wl.bpc > 8 and wl.w % 8 == 0  # rows of whole vectors
    if mode == "exact" and pitch:
        if vectors and pitch % 8 == 0 and x0 % 8 == 0:
            return "mapped_step", ("stage1_u16_mapped", "mapped_combine"), MAPPED_SOURCES
        return "view_step", ("view_stage1", "view_combine"), VIEW_SOURCES
    if mode == "exact":
        k = "stage1_u8" if wl.bpc == 8 else "stage1_u16"
        return k, (k,), STAGE1_SOURCES
    if mode == "cpu-order":
        if vectors:
            return ("cpu_order_step", ("stage1_u16_mapped",) + CPU_ORDER_KERNELS[1:],
                    CPU_ORDER_SOURCES + [os.path.join(CSRC, "stage1_mapped.hip")])
        if pitch:
            return ("cpu_order_step", ("gather_view",) + CPU_ORDER_KERNELS,
                    CPU_ORDER_SOURCES + [os.path.join(CSRC, "plane_views.hip")])
        return "cpu_order_step", CPU_ORDER_KERNELS, CPU_ORDER_SOURCES
    if mode == "psnr-int":
        return "psnr_int_step", ("view_stage1", "view_combine"), VIEW_SOURCES
    if mode == "yuv420":
        return "psnr_int_yuv420_step", ("views_stage1", "views_combine"), VIEW_SOURCES
    if mode == "hvs-sum":
        return "float_sum_step", FLOAT_SUM_KERNELS, FLOAT_SUM_SOURCES
    return "host_step", ("stage1_u16", "stage2_combine"), HOST_SOURCES
UNIT_POWER = (2, 1, 1, 2, 2)  # noise, ref1, dist1, ref2, dist2: units 1/s^power
STAMP_EVERY = 8  # exact mode: steps per stage-1 dispatch timed with its own events
MIN_STAMPED = 8  # ... but at least this many stamped dispatches in a short run


def stamp_interval(steps: int) -> int:
    """Steps per stamped stage-1 dispatch: one in STAMP_EVERY, or more often
    in a short run so that at least MIN_STAMPED timed dispatches are stamped
    (every one when there are fewer than 2 * MIN_STAMPED steps)."""
    return max(1, min(STAMP_EVERY, steps // MIN_STAMPED))


def stamped_steps(steps: int) -> list:
    """The timed steps (counted from 0) whose stage-1 dispatch is stamped:
    one in stamp_interval(steps), from the middle of the first interval."""
    every = stamp_interval(steps)
    phase = every // 2 if steps > every // 2 else 0
    return [j for j in range(steps) if j % every == phase]


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    p.add_argument("--gpus", type=int, default=1)
    # Under sustained load the pass runs slower for its first tens of
    # milliseconds while the power manager settles (about 190 us per batch
    # at first, 156 us after ~55 ms); 300 warm-up steps (~55 ms) get past
    # that, and the timed steps measure steady streaming.
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--workload", type=int, default=None,
                   help="workload number (default 5, 3840x2160 16-bit; 2, 1920x1080 10-bit, for yuv420)")
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle leg (and with it the parity gate); for profiler runs")
    p.add_argument("--input-cache", default=None, metavar="DIR",
                   help="keep the generated batch as .npy files in DIR and reuse them")
    p.add_argument("--planes", type=int, default=32,
                   help="hvs-sum mode: 3840x2160 term buffers per step")
    p.add_argument("--mode", choices=("exact", "cpu-order", "psnr-int", "yuv420", "host", "hvs-sum"), default="exact",
                   help="exact: the exact sums (default); cpu-order: also the CPU's rounding past 2^53; "
                        "psnr-int: the integer psnr twin; yuv420: the integer psnr twin on the Y, U and V "
                        "planes of planar 4:2:0 frames; host: the exact sums of a batch in pinned host "
                        "memory, uploads overlapped with the reduction; hvs-sum: the psnr_hvs running float "
                        "sum of psnr_hvs-like term buffers")
    p.add_argument("--streams", type=int, default=1,
                   help="streams the steps alternate over (step i on stream i %% N, each with its own "
                        "workspace): with more than one, consecutive steps overlap as in a pipeline of "
                        "batches, and a kernel's timed duration includes the overlap")
    p.add_argument("--pitch", type=int, default=0, metavar="SAMPLES",
                   help="exact, cpu-order and psnr-int modes: keep the planes resident with rows of SAMPLES samples "
                        "(>= w; the frame inside the first w of each row) and reduce them through the "
                        "plane-view entry points (default: contiguous)")
    p.add_argument("--x0", type=int, default=0, metavar="SAMPLES",
                   help="with --pitch: the frame starts SAMPLES samples into each row (pitch >= x0 + w)")
    p.add_argument("--frames-per-upload", type=int, default=4,
                   help="host mode: frames per upload")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                   help="after the timed steps, run 3 elementwise kernels that each read and "
                        "write MIB MiB (the known-size kernel that scales the HBM counters)")
    return p.parse_args(argv)


def kernel_source_sha256(paths=tuple(STAGE1_SOURCES)) -> str:
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def stored_traffic(kernel: str, workload: str, sources=tuple(STAGE1_SOURCES)):
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
    if fields.get("kernel_source_sha256") != kernel_source_sha256(sources):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000  # hipEventDisableSystemFence (hip_runtime_api.h)


class HipEvents:
    """Timing events from the HIP runtime torch and libvqx share."""

    def __init__(self, runtime: ctypes.CDLL):
        self.rt = runtime
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.rt.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
        self.rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.rt.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, flags: int = 0) -> int:
        ev = ctypes.c_void_p()
        if self.rt.hipEventCreateWithFlags(ctypes.byref(ev), flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")
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


def _oracle_o1_o2(ref, dist, bpc, threads):
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    n = ref.shape[0]
    with ThreadPoolExecutor(threads) as ex:
        o2 = list(ex.map(lambda f: oracle.exact_frame_sums(ref[f], dist[f]), range(n)))
        o1 = list(ex.map(lambda f: oracle.seq_frame_sums(ref[f], dist[f], bpc), range(n)))
    return o1, o2


def gate_exact(ref, dist, bpc, noise, moments, concl, threads):
    """The device's exact sums of the last batch, and the library's
    conclusion of them, against both oracles."""
    import oracle

    nframes, h, w = ref.shape
    o1, o2 = _oracle_o1_o2(ref, dist, bpc, threads)
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
    return parity


def gate_cpu_order(ref, dist, bpc, exact, cpu, concl, threads):
    """The last batch of the CPU-order mode: exact sums equal the exact
    oracle, the CPU-order sums equal the CPU's sequential doubles bit for bit
    on every frame, and the library's conclusion of them the CPU's scores."""
    import oracle

    nframes, h, w = ref.shape
    o1, o2 = _oracle_o1_o2(ref, dist, bpc, threads)
    s = 1 << (bpc - 8)
    failures = []
    past53 = 0
    for f in range(nframes):
        fails = []
        if [int(v) for v in exact[f]] != [int(v) for v in o2[f]]:
            fails.append("exact sums")
        for k in range(5):
            want = float(o1[f][k]) * float(s ** UNIT_POWER[k])
            if float(cpu[f][k]) != want or int(cpu[f][k]) != int(want):
                fails.append(f"output {k}: device {int(cpu[f][k])} CPU {int(want)}")
        want_concl = oracle.conclude_from_doubles(o1[f], w, h)
        if [concl[f, 0]] + list(concl[f, 2:]) != list(want_concl):
            fails.append("conclusion")
        if fails:
            failures.append((f, fails))
        past53 += sum(1 for v in o2[f] if int(v) >= oracle.TWO53)
    parity = {"frames": nframes, "failures": len(failures), "outputs_past_2^53": past53,
              "rule": "exact integers; the CPU-order sums bit-identical to the sequential doubles "
                      "on every frame and output"}
    if failures:
        parity["first_failure"] = str(failures[0])
    return parity


def _psnr_int_planes(ref, dist, planes, w, h):
    """(plane index, frame, ref view, dist view, pw, ph) of every plane of the
    batch: the luma pair itself, or the three planes of planar frames."""
    nframes = ref.shape[0]
    if planes is None:
        return [(0, f, ref[f], dist[f], w, h) for f in range(nframes)]
    out = []
    for p, (off, pw, ph) in enumerate(planes):
        for f in range(nframes):
            out.append((p, f, ref[f, off:off + pw * ph].reshape(ph, pw), dist[f, off:off + pw * ph].reshape(ph, pw),
                        pw, ph))
    return out


def gate_psnr_int(ref, dist, bpc, planes, w, h, last, concl):
    """The integer noise of every plane and frame of the last step against O3,
    and the library's conclusion of it against O3's."""
    import oracle

    nframes = ref.shape[0]
    failures = []
    for row, (p, f, r, d, pw, ph) in enumerate(_psnr_int_planes(ref, dist, planes, w, h)):
        want = oracle.int_noise(r, d)
        got = int(last[p * nframes + f])
        if got != want:
            failures.append((p, f, f"device {got} != exact {want}"))
        elif concl[row, 1] != oracle.int_psnr_db(want, pw, ph, bpc):
            failures.append((p, f, "conclusion"))
    parity = {"frames": nframes, "planes": 1 if planes is None else len(planes), "failures": len(failures),
              "rule": "exact integers; the conclusion bit-identical to the oracle's"}
    if failures:
        parity["first_failure"] = str(failures[0])
    return parity


def time_oracle_psnr_int(ref, dist, bpc, planes, w, h, threads):
    """O3 (numpy int64 sums of squared differences), one plane of one frame
    per task, over a bounded sample of the batch."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    work = _psnr_int_planes(ref, dist, planes, w, h)
    t = time.perf_counter()
    oracle.int_noise(work[0][2], work[0][3])
    one = max(time.perf_counter() - t, 1e-6)
    passes = max(1, min(50, int(12.0 / (one * len(work)))))
    items = [x for _ in range(passes) for x in work]
    t = time.perf_counter()
    with ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda x: oracle.int_noise(x[2], x[3]), items))
    wall = time.perf_counter() - t
    frames = passes * ref.shape[0]
    return {
        "value": round(frames / wall, 3), "unit": "frames/s", "cores": threads, "kind": "oracle",
        "sample": f"{passes} passes over the {ref.shape[0]} frames of the batch "
                  f"({'all three planes' if planes is not None else 'the plane pair'}), O3 "
                  "(numpy int64), one plane of one frame per task",
    }


def time_oracle(ref, dist, bpc, bytes_per_frame, threads):
    """The oracle as it stands (the CPU's sequential double loop), one frame
    per task on `threads` threads, over a bounded sample of the batch."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle

    nframes, h, w = ref.shape
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
    return {
        "value": round(fps, 3), "unit": "frames/s", "cores": threads, "kind": "oracle",
        "sample": f"{passes} passes over the {nframes} frames of the batch ({len(work)} frames of "
                  f"{w}x{h} at {bpc} bits), the C sequential-double oracle, one frame per task",
        "gbs": round(fps * bytes_per_frame / 1e9, 3),
        "single_thread_frames_per_s": round(1.0 / one, 3),
    }


def past53_bytes(ref, dist, bpc):
    """Bytes the CPU-order maps pass must read again for this batch.

    Per frame and square sum, the frame's whole 16-byte vectors are cut into
    chunks of 2048 (the few samples before the first and after the last whole
    vector count with chunk 0).  A chunk is read again, one plane for a sum
    of squares of one plane and both for the noise, when the running sum
    passes 2^53 units by its end, unless its terms cannot round: it starts
    past 2^53 inside one binade [2^e, 2^(e+1)) that its exact end stays in,
    and every one of its terms is a multiple of 2^(e-52).  Plain numpy and
    Python ints over the batch (float32 squares read back as integers); no
    part of the library or the oracle."""
    import numpy as np

    if bpc == 8:
        return 0
    nframes, h, w = ref.shape
    pixels = w * h
    table = (np.arange(65536, dtype=np.float32) ** 2).astype(np.uint64)
    two53 = 1 << 53
    chunk = 8 * 2048
    total = 0
    for f in range(nframes):
        e0, e1 = f * pixels, (f + 1) * pixels
        vb, ve = -(-e0 // 8), e1 // 8
        if vb >= ve:
            continue
        head, tail = vb * 8 - e0, e1 - ve * 8
        r = ref[f].reshape(-1)
        d = dist[f].reshape(-1)
        diff = np.abs(r.astype(np.float32) - d.astype(np.float32))
        kinds = ((np.rint(diff * diff).astype(np.uint64), 2), (table[r], 1), (table[d], 1))
        for terms, planes in kinds:
            if int(terms.sum()) < two53:
                continue
            body = terms[head:pixels - tail]
            starts = np.arange(0, body.size, chunk)
            sums = [int(v) for v in np.add.reduceat(body, starts)]
            ors = [int(v) for v in np.bitwise_or.reduceat(body, starts)]
            edge = np.concatenate((terms[:head], terms[pixels - tail:]))
            sums[0] += int(edge.sum())
            ors[0] |= int(np.bitwise_or.reduce(edge)) if edge.size else 0
            p = 0
            for c, (s, o) in enumerate(zip(sums, ors)):
                if p + s >= two53:
                    e = max(p, two53).bit_length() - 1
                    one_binade = p + s < (1 << (e + 1))
                    aligned = o & ((1 << (e - 52)) - 1) == 0
                    if not (p >= two53 and one_binade and aligned):
                        vectors = min(2048, (ve - vb) - c * 2048)
                        total += vectors * 16 * planes
                p += s
    return total


def measure_read_ceiling(L, hip, torch, bufs, wl, ws, ws_bytes, st, stage1_ms, alg_bytes, n):
    """The read time of stage 1's access pattern: the library's read probe
    (stage 1's grid, chunks and loads, no arithmetic) dispatched n times after
    20 untimed ones, alternating the two batch copies, each dispatch stamping
    its own events."""
    warm = 20
    evs = [(hip.create(HIP_EVENT_DISABLE_SYSTEM_FENCE), hip.create(HIP_EVENT_DISABLE_SYSTEM_FENCE))
           for _ in range(warm + n)]
    for j, (b, e) in enumerate(evs):
        r, d = bufs[j % 2]
        rc = L.vqx_read_probe_timed(r.data_ptr(), d.data_ptr(), wl.w, wl.h, wl.bpc, wl.nframes, ws.data_ptr(),
                                    ws_bytes, st, b, e)
        if rc != 0:
            raise RuntimeError(f"vqx_read_probe_timed: status {rc}")
    torch.cuda.synchronize()
    ms = [hip.elapsed_ms(b, e) for b, e in evs[warm:]]
    for b, e in evs:
        hip.destroy(b)
        hip.destroy(e)
    probe_ms = statistics.fmean(ms)
    gbs = alg_bytes / (probe_ms * 1e-3) / 1e9
    return {
        "kernel": "read_probe (stage 1's grid, chunks and 16-byte loads; an XOR of every word, no arithmetic)",
        "dispatches": n,
        "us_mean": round(probe_ms * 1e3, 2),
        "GBps": round(gbs, 1),
        "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
        "stage1_frac_of_ceiling": round(probe_ms / stage1_ms, 4),
    }


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


def run_host_mode(args, np, torch, vqx, wl, ref_np, dist_np, t_gen):
    """The host-fed mode: every step reduces the whole batch from pinned
    host memory (vqx_plane_stats_host_ws returns when it is done), so a
    step's wall time is the PCIe-inclusive time.  Also times a plain upload
    of the same bytes (two hipMemcpyAsync calls, no reduction) for the link
    rate this host reaches."""
    w, h, bpc, nframes = wl.w, wl.h, wl.bpc, wl.nframes
    dev = torch.device("cuda:0")
    L = vqx.lib()
    hip = HipEvents(vqx.hip_runtime())
    r = torch.from_numpy(ref_np).pin_memory()
    d = torch.from_numpy(dist_np).pin_memory()
    out = torch.zeros(5 * nframes, dtype=torch.int64, pin_memory=True)
    out_dev = hip.device_pointer(out.data_ptr())
    fpu = args.frames_per_upload
    ws_bytes = vqx.plane_stats_host_workspace_bytes(w, h, bpc, fpu)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    copy = torch.cuda.Stream(dev)  # default priority
    history = np.zeros((args.warmup + args.steps, 5 * nframes), dtype=np.int64)

    def step(i):
        rc = L.vqx_plane_stats_host_ws(r.data_ptr(), d.data_ptr(), w, h, bpc, nframes, fpu, out_dev,
                                       out_dev + 8 * nframes, ws.data_ptr(), ws_bytes, st, copy.cuda_stream)
        if rc != 0:
            raise vqx.VqxError(rc, "vqx_plane_stats_host_ws")
        history[i] = out.numpy()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    times = []
    for i in range(args.warmup, args.warmup + args.steps):
        t = time.perf_counter()
        step(i)
        times.append(time.perf_counter() - t)
    elapsed = time.perf_counter() - t0
    if not np.all(history == history[-1]):
        print("the steps disagree", file=sys.stderr)
        return 1

    # the link alone: the same bytes uploaded into device memory, no kernels
    dst_r = torch.empty(r.shape, dtype=r.dtype, device=dev)
    dst_d = torch.empty(d.shape, dtype=d.dtype, device=dev)
    copy_s = []
    for _ in range(5):
        torch.cuda.synchronize()
        t = time.perf_counter()
        dst_r.copy_(r, non_blocking=True)
        dst_d.copy_(d, non_blocking=True)
        torch.cuda.synchronize()
        copy_s.append(time.perf_counter() - t)
    link_gbs = 2 * ref_np.nbytes / min(copy_s) / 1e9

    upload = 2 * ref_np.nbytes
    mean_s = statistics.fmean(times)
    achieved = upload / mean_s / 1e9
    result = {
        "metric": METRIC_HOST,
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
                        f"{'uint8' if bpc == 8 else 'uint16'} ({wl.recipe}), in pinned host memory",
            "w": w, "h": h, "bpc": bpc, "nframes": nframes, "mode": "host",
            "frames_per_upload": fpu, "bytes_per_step": upload,
        },
        "roofline": {
            "bound": "pcie",
            "kernel": "host-fed step (H2D uploads overlapped with stage1_u16 + stage2_combine)",
            "achieved": round(achieved, 2),
            "peak": PCIE_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PCIE_PEAK_GBS, 4),
            "traffic": None,
            "step_ms_mean": round(mean_s * 1e3, 3),
            "step_ms_median": round(statistics.median(times) * 1e3, 3),
            "algorithmic_bytes_per_launch": upload,
            "plain_upload_gbs_this_host": round(link_gbs, 2),
            "frac_of_plain_upload": round(achieved / link_gbs, 4),
        },
        "generation_s": round(t_gen, 1),
    }

    if not args.no_cpu_baseline:
        threads = cpu_threads()
        last = history[-1]
        concl = vqx.conclude_batch(last[:nframes], last[nframes:].reshape(nframes, 4), w, h, bpc, 0.0)
        result["parity"] = gate_exact(ref_np, dist_np, bpc, last[:nframes], last[nframes:].reshape(nframes, 4),
                                      concl, threads)
        result["cpu_baseline"] = time_oracle(ref_np, dist_np, bpc, wl.bytes_per_frame, threads)
        if result["parity"]["failures"]:
            print(json.dumps({"error": "timed batch does not match the oracle", "parity": result["parity"]}),
                  file=sys.stderr)
            return 1
    print(json.dumps(result), flush=True)
    return 0


class Mode:
    """What one bench step runs, per mode: the sums per slot (int64), the
    enqueue of one step, the host conclusion of one slot, the step's
    algorithmic bytes and the gate of the last step."""


def make_mode(args, vqx, L, hip, np, torch, dev, st, wl, ref_np, dist_np, planes, bufs):
    """Builds the Mode of ``args.mode``.  Device outputs are pinned host
    memory written through its device mapping; ``bufs`` holds the two
    resident copies of the batch."""
    w, h, bpc, nframes = wl.w, wl.h, wl.bpc, wl.nframes
    m = Mode()
    m.name = args.mode
    m.per_step_events = args.mode == "exact" and not args.pitch
    kernel, step_kernels, m.sources = step_plan(args.mode, wl, args.pitch, args.x0 if args.pitch else 0)
    if args.mode == "exact" and args.pitch:
        m.width = 5 * nframes
        m.ws_bytes = vqx.plane_view_workspace_bytes(w, h, bpc, nframes)
        m.metric = METRIC
        m.kernel = kernel
        m.kernel_label = f"{kernel} ({', '.join(step_kernels)})"
        m.alg_bytes = wl.bytes_per_frame * nframes
    elif args.mode == "exact":
        m.width = 5 * nframes
        m.ws_bytes = vqx.plane_stats_workspace_bytes(w, h, bpc, nframes)
        m.metric = METRIC
        m.kernel = kernel
        m.kernel_label = m.kernel
        m.alg_bytes = wl.bytes_per_frame * nframes
    elif args.mode == "cpu-order":
        m.width = 10 * nframes
        m.ws_bytes = (vqx.plane_stats_view_cpu_order_workspace_bytes(w, h, bpc, nframes) if args.pitch
                      else vqx.plane_stats_cpu_order_workspace_bytes(w, h, bpc, nframes))
        m.metric = METRIC_CPU_ORDER
        m.kernel = kernel
        m.kernel_label = f"{kernel} ({', '.join(step_kernels)})"
        m.alg_bytes = wl.bytes_per_frame * nframes + past53_bytes(ref_np, dist_np, bpc)
    elif args.mode == "psnr-int":
        m.width = nframes
        m.ws_bytes = vqx.plane_view_workspace_bytes(w, h, bpc, nframes)
        m.metric = METRIC_PSNR_INT
        m.kernel = kernel
        m.kernel_label = f"{kernel} (view_stage1 integer noise, view_combine)"
        m.alg_bytes = wl.bytes_per_frame * nframes
    else:  # yuv420
        m.width = 3 * nframes
        m.ws_bytes = vqx.planes_workspace_bytes([(pw, ph) for _, pw, ph in planes], bpc, nframes)
        # the three planes of each batch copy as views of its frames
        fs = ref_np.shape[1]
        m.plane_arrays = []
        for r, d in bufs:
            pairs = [(torch.as_strided(r, (nframes, ph, pw), (fs, pw, 1), off),
                      torch.as_strided(d, (nframes, ph, pw), (fs, pw, 1), off)) for off, pw, ph in planes]
            m.plane_arrays.append(vqx.plane_pairs(pairs, bpc)[0])
        m.metric = METRIC_YUV420
        m.kernel = kernel
        m.kernel_label = f"{kernel} (views_stage1 integer noise, views_combine; Y, U, V in one launch each)"
        m.alg_bytes = 2 * ref_np.shape[1] * wl.bytes_per_sample * nframes
    m.ws = torch.empty(m.ws_bytes, dtype=torch.uint8, device=dev)
    return m


def calibrate_copy(torch, dev, mib):
    """Three runs of a kernel that reads exactly `mib` MiB and writes exactly
    as much (the scale for the profiler's byte counters)."""
    n = mib * (1 << 20)
    src = torch.ones(n // 4, dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.bitwise_not(src, out=dst)
    torch.cuda.synchronize()
    del src, dst


def run_hvs_sum(args, np, torch, synth, vqx):
    """hvs-sum mode: each step sums ``args.planes`` psnr_hvs-like term
    buffers of a 3840x2160 luma plane (548 x 308 blocks of 64 terms) with
    vqx_float_running_sums_ws; two copies of the batch alternate, resident
    in HBM.  The step is timed with HIP events around the timed region; the
    roofline is the whole step against one read of the terms."""
    dev = torch.device("cuda:0")
    bw, bh = synth.HVS_4K_BLOCKS
    n = bw * bh * 64
    t_gen = time.perf_counter()
    terms_np = synth.hvs_like_terms(bw * bh, args.planes, seed=1397)
    t_gen = time.perf_counter() - t_gen
    bufs = [torch.from_numpy(terms_np).to(dev) for _ in range(2)]
    out = torch.empty(args.planes, dtype=torch.float32, device=dev)
    ws_bytes = vqx.float_sum_workspace_bytes(n, args.planes)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    L = vqx.lib()
    hip = HipEvents(vqx.hip_runtime())
    st = torch.cuda.current_stream(dev).cuda_stream
    torch.cuda.synchronize()

    def step(i):
        b = bufs[i % 2]
        rc = L.vqx_float_running_sums_ws(b.data_ptr(), n, args.planes, out.data_ptr(), ws.data_ptr(), ws_bytes, st)
        if rc != 0:
            raise vqx.VqxError(rc, "vqx_float_running_sums_ws")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    e0, e1 = hip.create(), hip.create()
    t0 = time.perf_counter()
    hip.record(e0, st)
    for i in range(args.steps):
        step(args.warmup + i)
    hip.record(e1, st)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gpu_ms = hip.elapsed_ms(e0, e1) / args.steps
    hip.destroy(e0)
    hip.destroy(e1)
    got = out.cpu().numpy()
    if args.calibrate_copy:
        calibrate_copy(torch, dev, args.calibrate_copy)

    alg = 4 * n * args.planes  # one read of the terms
    achieved = alg / (gpu_ms * 1e-3) / 1e9
    kernel, step_kernels, sources = step_plan("hvs-sum", None)
    wname = f"3840x2160x{args.planes}_hvs"
    traffic = stored_traffic(kernel, wname, tuple(sources))
    result = {
        "metric": METRIC_HVS_SUM,
        "value": round(args.steps * args.planes / elapsed, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 running sum (integer two-state maps inside a binade, binary32 adds where it crosses)",
        "data": "synthetic",
        "config": {
            "workload": (f"{args.planes} psnr_hvs-like term buffers of a 3840x2160 luma plane "
                         f"({bw}x{bh} blocks of 64 float32 terms, {n} each, 17-31 % nonzero)"),
            "planes": args.planes, "terms_per_plane": n, "mode": "hvs-sum", "bytes_per_step": alg,
        },
        "roofline": {
            "bound": "hbm",
            "kernel": f"{kernel} ({', '.join(step_kernels)})",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": (f"profiles/{kernel}_{wname}_hbm_traffic.txt" if traffic is not None else None),
            "step_us_mean": round(gpu_ms * 1e3, 2),
            "timed_by": "HIP events around the timed steps, per step",
            "algorithmic_bytes_per_launch": alg,
        },
        "generation_s": round(t_gen, 1),
    }
    if not args.no_cpu_baseline:
        want = oracle_module().running_float_sums(terms_np)
        bad = int(np.count_nonzero(got.view(np.uint32) != want.view(np.uint32)))
        result["parity"] = {"planes": args.planes, "failures": bad,
                            "rule": "every running sum bit-identical to the sequential binary32 oracle"}
        threads = cpu_threads()
        result["cpu_baseline"] = time_oracle_float_sums(terms_np, threads)
        if bad:
            print(json.dumps({"error": "timed batch does not match the oracle", "parity": result["parity"]}),
                  file=sys.stderr)
            return 1
    print(json.dumps(result), flush=True)
    return 0


def oracle_module():
    import oracle
    return oracle


def time_oracle_float_sums(terms_np, threads):
    """O4 (the sequential binary32 sum in C) over the batch's planes, one
    plane per task on ``threads`` host threads, repeated to ~10 s."""
    import concurrent.futures
    oracle = oracle_module()
    planes = terms_np.shape[0]
    reps = 0
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as pool:
        while time.perf_counter() - t0 < 10.0 or reps == 0:
            list(pool.map(lambda k: oracle.running_float_sums(terms_np[k:k + 1]), range(planes)))
            reps += 1
    el = time.perf_counter() - t0
    t1 = time.perf_counter()
    oracle.running_float_sums(terms_np[:1])
    single = time.perf_counter() - t1
    return {"value": round(reps * planes / el, 1), "unit": "frames/s", "cores": threads, "kind": "oracle",
            "sample": f"{reps} passes over the {planes} planes of the batch, the C sequential binary32 sum, "
                      "one plane per task",
            "single_thread_frames_per_s": round(1.0 / single, 1)}


def main(argv=None):
    args = parse_args(argv)
    if args.workload is None:
        args.workload = 2 if args.mode == "yuv420" else 5
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
    if args.mode == "hvs-sum":
        return run_hvs_sum(args, np, torch, synth, vqx)
    dev = torch.device("cuda:0")
    wl = synth.WORKLOADS[args.workload]
    w, h, bpc, nframes = wl.w, wl.h, wl.bpc, wl.nframes

    t_gen = time.perf_counter()
    planes = None
    if args.mode == "yuv420":
        ref_np, dist_np, planes = synth.planar_yuv(args.workload, "420")
    else:
        ref_np, dist_np = load_or_generate(args.workload, args.input_cache)
    t_gen = time.perf_counter() - t_gen
    if args.mode == "host":
        if args.steps == 500 and args.warmup == 300:  # the defaults of the device-resident modes
            args.steps, args.warmup = 20, 3
        return run_host_mode(args, np, torch, vqx, wl, ref_np, dist_np, t_gen)

    # two resident copies of the batch, alternated step by step
    r0 = torch.from_numpy(ref_np).to(dev)
    d0 = torch.from_numpy(dist_np).to(dev)
    if args.pitch == w and not args.x0:
        args.pitch = 0
    if args.pitch:
        if args.mode not in ("exact", "cpu-order", "psnr-int") or args.x0 < 0 or args.pitch < args.x0 + w:
            print("--pitch needs --mode exact, cpu-order or psnr-int and a pitch >= x0 + w", file=sys.stderr)
            return 2
        x0 = args.x0

        def pitched(x):
            big = torch.zeros((nframes, h, args.pitch), dtype=x.dtype, device=dev)
            big[:, :, x0:x0 + w] = x
            return big[:, :, x0:x0 + w]
        bufs = [(pitched(r0), pitched(d0)), (pitched(r0), pitched(d0))]
        del r0, d0
    else:
        bufs = [(r0, d0), (r0.clone(), d0.clone())]
    rs = args.pitch or w  # row and frame strides of the resident planes, in samples
    fs = rs * h
    # Sums land directly in pinned host memory that the GPU writes through
    # (zero-copy): the last kernel of a step stores its few bytes per frame
    # there, and no copy kernel runs.  `depth` groups of slots, so that the
    # GPU always has several groups queued while the host concludes the
    # oldest one.
    group = 8
    depth = 4  # groups in flight: ~5 ms of queued work absorbs host hiccups
    nslots = depth * group
    stream = torch.cuda.current_stream(dev)
    st = stream.cuda_stream
    # every stream at the default priority
    side = [torch.cuda.Stream(device=dev) for _ in range(max(1, args.streams) - 1)]
    sts = [st] + [x.cuda_stream for x in side]
    nst = len(sts)
    hip = HipEvents(vqx.hip_runtime())
    L = vqx.lib()
    mode = make_mode(args, vqx, L, hip, np, torch, dev, st, wl, ref_np, dist_np, planes, bufs)
    width = mode.width
    sums = torch.zeros((nslots, width), dtype=torch.int64, pin_memory=True)
    sums_dev = [hip.device_pointer(sums[s].data_ptr()) for s in range(nslots)]
    sums_np = sums.numpy()
    ws, ws_bytes = mode.ws, mode.ws_bytes
    wss = [ws] + [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(nst - 1)]
    total = args.warmup + args.steps
    # exact mode: stage 1 of one step in every `every` stamps its own events
    # (a stamped dispatch costs the queue ~10 us of extra gaps, so stamping
    # every step of a long run would slow the stream it measures; a short
    # run stamps more often to keep the mean stable); other modes: events
    # around each group of steps
    every = stamp_interval(args.steps)
    # the stamps only time the dispatch, and the host never waits on them, so
    # they are made without the system-scope fence (a write-back of the L2s
    # that an ordinary event performs when it is reached)
    ev_begin = ({args.warmup + j: hip.create(HIP_EVENT_DISABLE_SYSTEM_FENCE) for j in stamped_steps(args.steps)}
                if mode.per_step_events else {})
    ev_end = {i: hip.create(HIP_EVENT_DISABLE_SYSTEM_FENCE) for i in ev_begin}
    ngroups = (total + group - 1) // group + 1
    ev_start = [hip.create() for _ in range(ngroups)] if not mode.per_step_events else []
    ev_done = [hip.create() for _ in range(ngroups)]
    ev_join = [hip.create() for _ in range(nst)]  # the other streams' ends of a group
    torch.cuda.synchronize()

    # The host conclusion allocates nothing: libvqx concludes from the pinned
    # sums into preallocated arrays, and each step's sums are copied in place
    # into a preallocated history (to check afterwards that every step gave
    # the same sums).  Allocating numpy temporaries per batch stalled the
    # host for up to tens of milliseconds after the batch generation.
    ncon = 6 if args.mode in ("exact", "cpu-order") else 2
    nrows = nframes * (3 if args.mode == "yuv420" else 1)
    concl = np.zeros((nslots, nrows, ncon), dtype=np.float64)
    concl_ptr = [concl[s].ctypes.data for s in range(nslots)]
    base_ptr = [sums[s].data_ptr() for s in range(nslots)]
    history = np.zeros((total, width), dtype=np.int64)
    plane_dims = [(w, h)] if planes is None else [(pw, ph) for _, pw, ph in planes]
    itemsize = 8

    # host time spent inside each step's library call (argument checks,
    # launches): the library's own per-call cost, which bounds the step of a
    # small batch
    call_s = np.zeros(total, dtype=np.float64)

    def enqueue(i):
        s = i % nslots
        r, d = bufs[i % 2]
        o = sums_dev[s]
        st = sts[i % nst]
        ws = wss[i % nst]
        t_call = time.perf_counter()
        if args.mode == "exact" and args.pitch:
            rc = L.vqx_plane_stats_view_ws(r.data_ptr(), rs, fs, d.data_ptr(), rs, fs, w, h, bpc, nframes,
                                           o, o + itemsize * nframes, ws.data_ptr(), ws_bytes, st)
        elif args.mode == "exact":
            rc = L.vqx_plane_stats_batch_ws_timed(r.data_ptr(), d.data_ptr(), w, h, bpc, nframes,
                                                  o, o + itemsize * nframes, ws.data_ptr(), ws_bytes,
                                                  st, ev_begin.get(i), ev_end.get(i))
        elif args.mode == "cpu-order" and args.pitch:
            rc = L.vqx_plane_stats_view_cpu_order_ws(r.data_ptr(), rs, fs, d.data_ptr(), rs, fs, w, h, bpc, nframes,
                                                     o, o + itemsize * nframes, o + itemsize * 5 * nframes,
                                                     o + itemsize * 6 * nframes, ws.data_ptr(), ws_bytes, st)
        elif args.mode == "cpu-order":
            rc = L.vqx_plane_stats_batch_cpu_order_ws(r.data_ptr(), d.data_ptr(), w, h, bpc, nframes,
                                                      o, o + itemsize * nframes, o + itemsize * 5 * nframes,
                                                      o + itemsize * 6 * nframes, ws.data_ptr(), ws_bytes, st)
        elif args.mode == "psnr-int":
            rc = L.vqx_psnr_int_view_ws(r.data_ptr(), rs, fs, d.data_ptr(), rs, fs, w, h, bpc, nframes,
                                        o, ws.data_ptr(), ws_bytes, st)
        else:
            rc = L.vqx_psnr_int_planes_ws(mode.plane_arrays[i % 2], len(planes), bpc, nframes, o, ws.data_ptr(),
                                          ws_bytes, st)
        call_s[i] = time.perf_counter() - t_call
        if rc != 0:
            raise vqx.VqxError(rc, f"libvqx entry point ({args.mode})")

    def conclude(steps, done):
        hip.synchronize(done)
        for i in steps:
            s = i % nslots
            if args.mode in ("exact", "cpu-order"):
                # the exact sums, or in the CPU-order mode the CPU's
                off = 5 * nframes if args.mode == "cpu-order" else 0
                rc = L.vqx_conclude_batch(base_ptr[s] + itemsize * off, base_ptr[s] + itemsize * (off + nframes),
                                          w, h, bpc, nframes, 0.0, concl_ptr[s])
                if rc != 0:
                    raise vqx.VqxError(rc, "vqx_conclude_batch")
            else:
                for p, (pw, ph) in enumerate(plane_dims):
                    rc = L.vqx_conclude_psnr_int_batch(base_ptr[s] + itemsize * p * nframes, pw, ph, bpc,
                                                       nframes, 0.0, concl_ptr[s] + 2 * itemsize * p * nframes)
                    if rc != 0:
                        raise vqx.VqxError(rc, "vqx_conclude_psnr_int_batch")
            history[i] = sums_np[s]

    def run(first, count):
        # step i uses slot i % nslots; a slot is reused only after the group
        # that last used it was concluded (at most `depth` groups in flight)
        groups = [list(range(a, min(a + group, first + count))) for a in range(first, first + count, group)]
        pending = []
        for steps in groups:
            if len(pending) == depth:
                conclude(*pending.pop(0))
            # a group starts on every stream after the start event and ends
            # when every stream has finished its steps of the group
            if not mode.per_step_events:
                hip.record(ev_start[steps[0] // group], st)
                for k in range(1, nst):
                    hip.wait(sts[k], ev_start[steps[0] // group])
            for i in steps:
                enqueue(i)
            for k in range(1, nst):
                hip.record(ev_join[k], sts[k])
                hip.wait(st, ev_join[k])
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

    if mode.per_step_events:
        step_ms = [hip.elapsed_ms(ev_begin[i], ev_end[i]) for i in ev_begin if i >= args.warmup]
    else:
        # device time per step, from the events around each timed group
        step_ms = []
        for a in range(args.warmup, total, group):
            g = a // group
            n = min(group, total - a)
            step_ms += [hip.elapsed_ms(ev_start[g], ev_done[g]) / n] * n
    for ev in list(ev_begin.values()) + list(ev_end.values()) + ev_start + ev_done + ev_join:
        hip.destroy(ev)

    # every step must have produced the same sums
    if not np.all(history == history[total - 1]):
        bad = int(np.nonzero(np.any(history != history[total - 1], axis=1))[0][0])
        print(f"step {bad} differs from the last step", file=sys.stderr)
        return 1
    last = history[total - 1]
    last_concl = concl[(total - 1) % nslots].copy()

    if args.calibrate_copy:
        calibrate_copy(torch, dev, args.calibrate_copy)

    bytes_per_frame = wl.bytes_per_frame
    bytes_per_step = ref_np[0].size * wl.bytes_per_sample * 2 * nframes
    mean_ms = statistics.fmean(step_ms)
    read_ceiling = None
    if args.mode == "exact" and not args.pitch:
        read_ceiling = measure_read_ceiling(L, hip, torch, bufs, wl, ws, ws_bytes, st, mean_ms,
                                            mode.alg_bytes, min(args.steps, 200))

    wname = (f"{w}x{h}x{nframes}_{bpc}bit" + ("_yuv420" if args.mode == "yuv420" else "")
             + (f"_pitch{args.pitch}" if args.pitch else "") + (f"_x{args.x0}" if args.pitch and args.x0 else ""))
    traffic = stored_traffic(mode.kernel, wname, tuple(mode.sources))
    achieved = mode.alg_bytes / (mean_ms * 1e-3) / 1e9

    out = {
        "metric": mode.metric,
        "value": round(args.steps * nframes / elapsed, 1),
        "unit": "frames/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32 squares, u64 sums" if args.mode in ("exact", "cpu-order") else "u32 squares, u64 sums",
        "data": "synthetic",
        "config": {
            "workload": f"{w}x{h} {bpc}-bit luma pair, {nframes} frames, "
                        f"{'uint8' if bpc == 8 else 'uint16'} ({wl.recipe})"
                        + (", as planar 4:2:0 frames (Y, U, V each drawn with the recipe at its size)"
                           if args.mode == "yuv420" else ""),
            "w": w, "h": h, "bpc": bpc, "nframes": nframes, "mode": args.mode,
            "streams": nst,
            "row_pitch": args.pitch or w,
            "x0": args.x0 if args.pitch else 0,
            "bytes_per_step": bytes_per_step,
            "hbm_gbs_whole_step": round(bytes_per_step * args.steps / elapsed / 1e9, 1),
        },
        "roofline": {
            "bound": "hbm",
            "kernel": mode.kernel_label,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "traffic_source": (f"profiles/{mode.kernel}_{wname}_hbm_traffic.txt (rocprofv3 --pmc FETCH_SIZE, then "
                               f"WRITE_SIZE, scaled by a copy kernel; taken for the same kernel source, not by "
                               f"this run)" if traffic is not None else None),
            "kernel_us_mean": round(mean_ms * 1e3, 2),
            "kernel_us_median": round(statistics.median(step_ms) * 1e3, 2),
            "kernel_us_min": round(min(step_ms) * 1e3, 2),
            "kernel_us_max": round(max(step_ms) * 1e3, 2),
            "timed_by": (f"HIP events stamped by {len(step_ms)} of the {args.steps} timed stage-1 dispatches "
                         f"(one in {every})" if mode.per_step_events else
                         f"HIP events around each group of {group} timed steps, per step"),
            "algorithmic_bytes_per_launch": mode.alg_bytes,
        },
        "generation_s": round(t_gen, 1),
        "host_call_us": {
            "mean": round(float(call_s[args.warmup:].mean()) * 1e6, 1),
            "median": round(float(np.median(call_s[args.warmup:])) * 1e6, 1),
            "what": "host time inside the step's library call (checks and launches), timed steps",
        },
    }
    if read_ceiling:
        out["read_ceiling"] = read_ceiling

    if not args.no_cpu_baseline:
        threads = cpu_threads()
        if args.mode == "cpu-order":
            exact = np.concatenate([last[:nframes, None], last[nframes:5 * nframes].reshape(nframes, 4)], 1)
            cpu = np.concatenate([last[5 * nframes:6 * nframes, None], last[6 * nframes:].reshape(nframes, 4)], 1)
            parity = gate_cpu_order(ref_np, dist_np, bpc, exact, cpu, last_concl, threads)
        elif args.mode == "exact":
            parity = gate_exact(ref_np, dist_np, bpc, last[:nframes], last[nframes:].reshape(nframes, 4),
                                last_concl, threads)
        else:
            parity = gate_psnr_int(ref_np, dist_np, bpc, planes, w, h, last, last_concl)
        if args.mode in ("exact", "cpu-order"):
            out["cpu_baseline"] = time_oracle(ref_np, dist_np, bpc, bytes_per_frame, threads)
        else:
            out["cpu_baseline"] = time_oracle_psnr_int(ref_np, dist_np, bpc, planes, w, h, threads)
        out["parity"] = parity
        if parity["failures"]:
            print(json.dumps({"error": "timed batch does not match the oracle", "parity": parity}),
                  file=sys.stderr)
            return 1
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
