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
