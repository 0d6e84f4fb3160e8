"""The committed rocprofv3 summaries belong to the sources in the tree.

Each summary under profiles/ records the command that made it and the
SHA-256 of the kernel sources of that command's step.  The bench reports a
summary's counter traffic only while that hash matches; this test makes a
stale summary fail here, so that none is committed for sources that have
moved on.  It also checks that each counter summary has its kernel trace
beside it, taken for the same sources.
"""

from __future__ import annotations

import glob
import os
import re

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SUMMARIES = sorted(glob.glob(os.path.join(ROOT, "profiles", "*.txt")))


def _fields(path):
    text = open(path).read()
    sha = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    cmd = re.search(r"^command[a-z_]*:.*?\bbench\.py (.*)$", text, re.M)
    return (sha.group(1) if sha else None), (cmd.group(1).split() if cmd else None)


def test_there_are_summaries():
    assert len(SUMMARIES) >= 20


@pytest.mark.parametrize("path", SUMMARIES, ids=[os.path.basename(p) for p in SUMMARIES])
def test_summary_matches_the_sources(path):
    sha, toks = _fields(path)
    assert sha is not None, "no kernel_source_sha256 line"
    assert toks is not None, "no bench.py command line"

    def opt(name, default):
        return toks[toks.index(name) + 1] if name in toks else default

    wl = synth.WORKLOADS[int(opt("--workload", "5"))]
    pitch = int(opt("--pitch", "0")) or None
    _, _, sources = bench.step_plan(opt("--mode", "exact"), wl, pitch, int(opt("--x0", "0")))
    assert bench.kernel_source_sha256(sources) == sha, "taken for other sources: regenerate it with bench_profile.py"


@pytest.mark.parametrize("path", [p for p in SUMMARIES if p.endswith("_hbm_traffic.txt")],
                         ids=lambda p: os.path.basename(p))
def test_counter_summary_has_its_trace(path):
    trace = path[: -len("_hbm_traffic.txt")] + "_kernel_trace.txt"
    assert os.path.exists(trace)
    assert _fields(trace)[0] == _fields(path)[0]
