"""The bench's step plans name kernels that the listed sources define (CPU).

bench.py and bench_profile.py find a mode's kernels in rocprofv3 traces and
its stored counter summaries by these names and source hashes, so a renamed
kernel or a moved source would silently null the bench line's HBM traffic.
"""

from __future__ import annotations

import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402

PLANS = [(m, wl, p) for m in ("exact", "cpu-order", "psnr-int", "host") for wl in (2, 5) for p in (0, 3904, 3844)
         if not (m in ("psnr-int", "host") and p)] + [("yuv420", 2, 0)]


@pytest.mark.parametrize("mode,n,pitch", PLANS)
def test_step_plan_names_defined_kernels(mode, n, pitch):
    wl = synth.WORKLOADS[n]
    kernel, step_kernels, sources = bench.step_plan(mode, wl, pitch)
    assert kernel and step_kernels
    text = ""
    for path in sources:
        assert os.path.exists(path), path
        with open(path) as f:
            text += f.read()
    # every source the step's kernels come from: the listed ones plus the
    # launches they make into other files of the library
    with open(os.path.join(ROOT, "exact_reductions_amd", "csrc", "plane_stats.hip")) as f:
        text += f.read()
    for k in step_kernels:
        assert re.search(r"void\s+" + re.escape(k) + r"\s*\(", text), f"{mode}: kernel {k} not defined"


def test_pitched_plans_follow_the_in_place_rule():
    wl = synth.WORKLOADS[5]
    assert bench.step_plan("exact", wl, 3904)[1][0] == "stage1_u16_mapped"   # whole aligned vectors
    assert bench.step_plan("exact", wl, 3844)[1][0] == "view_stage1"         # rows at other offsets
    assert bench.step_plan("cpu-order", wl, 3904)[1][0] == "stage1_u16_mapped"
    assert bench.step_plan("cpu-order", wl, 3844)[1][0] == "stage1_u16_mapped"  # rows at varying phases
    assert bench.step_plan("cpu-order", synth.WORKLOADS[1], 600)[1][0] == "gather_view"  # one-byte samples
    assert bench.step_plan("exact", synth.WORKLOADS[1], 600)[1][0] == "view_stage1"  # one-byte samples
    # a frame 4 samples into rows of whole vectors: in place for the CPU-order form only
    assert bench.step_plan("cpu-order", wl, 3904, 4)[1][0] == "stage1_u16_mapped"
    assert bench.step_plan("exact", wl, 3904, 4)[1][0] == "view_stage1"
    assert bench.step_plan("exact", wl, 3904, 8)[1][0] == "stage1_u16_mapped"


def test_stamping_events_flag_is_the_runtimes():
    """The bench's stamping events are made without the system-scope fence:
    its flag must be the HIP runtime's own hipEventDisableSystemFence."""
    header = "/opt/rocm/include/hip/hip_runtime_api.h"
    if not os.path.exists(header):
        pytest.skip("no ROCm headers")
    with open(header) as f:
        m = re.search(r"#define\s+hipEventDisableSystemFence\s+(0x[0-9a-fA-F]+)", f.read())
    assert m, "hipEventDisableSystemFence not defined in the HIP header"
    assert bench.HIP_EVENT_DISABLE_SYSTEM_FENCE == int(m.group(1), 16)


@pytest.mark.parametrize("steps", [1, 3, 8, 15, 16, 20, 63, 64, 65, 500])
def test_short_runs_stamp_enough_dispatches(steps):
    """At least MIN_STAMPED of the timed dispatches are stamped (all of them
    in a run shorter than that), and never more often than needed."""
    stamped = bench.stamped_steps(steps)
    assert len(stamped) >= min(steps, bench.MIN_STAMPED)
    assert all(0 <= j < steps for j in stamped) and stamped == sorted(set(stamped))
    assert 1 <= bench.stamp_interval(steps) <= bench.STAMP_EVERY
