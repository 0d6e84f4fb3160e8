"""The stage-1 group forms against the oracle, on an MI355X (marked gpu).

Stage 1 reads each lane's vectors in groups; a wave whose group's samples are
all bright (at least 49152, depths 13..16) or all small (below 4096, depths up
to 12) adds them in a cheaper form, any other group in the general form.
These batches mix the forms inside chunks, waves and frames, put samples on
both sides of each test's threshold, and fill groups with the largest terms
each form's budget allows.  Every sum must equal the exact integer (O2), and
the CPU's doubles (O1) below 2^53 units, frame by frame.
"""

from __future__ import annotations

import numpy as np
import pytest

import synth
from test_parity_gpu import check, device_sums

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _sprinkle(planes, rng, rate, values):
    """Set a fraction ``rate`` of the samples of each plane to draws from
    ``values`` (an array), at random positions."""
    out = []
    for p in planes:
        p = p.copy()
        mask = rng.random(p.shape) < rate
        p[mask] = rng.choice(values, size=int(mask.sum()))
        out.append(p)
    return out


@pytest.mark.parametrize("bpc", [13, 16])
@pytest.mark.parametrize("rate", [0.0, 2e-5, 3e-4])
def test_bright_groups_mixed_with_general_ones(bpc, rate):
    """Bright frames (49152..65535) with a few samples below 49152.  A wave's
    group holds 4096 samples, so with rate 2e-5 about one group in twelve
    falls back to the general form, with 3e-4 about seven in ten."""
    rng = np.random.Generator(np.random.PCG64(700 + bpc + int(rate * 1e6)))
    ref, dist = synth.uniform_planes(1024, 512, 3, 16, seed=710 + bpc, lo=49152, hi=65535)
    low = np.array([0, 1, 4095, 4096, 4097, 46340, 46341, 49151], dtype=np.uint16)
    ref, dist = _sprinkle((ref, dist), rng, rate, low)
    noise, moments = device_sums(ref, dist, bpc, entry="workspace_ff", prefill=-1)
    check(ref, dist, bpc, noise, moments)


@pytest.mark.parametrize("bpc", [9, 12])
@pytest.mark.parametrize("rate", [0.0, 2e-5, 3e-4])
def test_small_groups_mixed_with_general_ones(bpc, rate):
    """Small frames (0..4095 in the container) with a few samples of 4096 and
    above, up to 65535 (legal: not an error at any depth)."""
    rng = np.random.Generator(np.random.PCG64(800 + bpc + int(rate * 1e6)))
    ref, dist = synth.uniform_planes(1024, 512, 3, 16, seed=810 + bpc, lo=0, hi=4095)
    high = np.array([4096, 4097, 8191, 46341, 49152, 65535], dtype=np.uint16)
    ref, dist = _sprinkle((ref, dist), rng, rate, high)
    noise, moments = device_sums(ref, dist, bpc, entry="workspace_ff", prefill=-1)
    check(ref, dist, bpc, noise, moments)


@pytest.mark.parametrize("ref_value,dist_value,bpc", [
    (65535, 49152, 16),   # largest noise term of the bright form, 16383^2, in every slot
    (49152, 65535, 16),
    (49152, 49152, 16),   # smallest bright squares, zero noise
    (65535, 65535, 13),   # largest squares, 4294836224 each
    (49151, 65535, 16),   # one below the bright test: every group general
    (4095, 0, 12),        # largest small squares
    (0, 4095, 10),
    (4096, 0, 12),        # one above the small test: every group general
])
def test_form_budgets_on_constant_planes(ref_value, dist_value, bpc):
    """Constant planes fill every group with the same largest (or boundary)
    terms; the closed forms w*h*q(d) and w*h*q(v) hold exactly."""
    ref, dist = synth.constant_pair(2048, 1024, 2, bpc, ref_value, dist_value)
    noise, moments = device_sums(ref, dist, bpc, entry="workspace_ff", prefill=-1)
    check(ref, dist, bpc, noise, moments)


@pytest.mark.parametrize("bpc,lo,hi", [(16, 49152, 65535), (12, 0, 4095)])
@pytest.mark.parametrize("w,h,nframes", [(1031, 577, 3), (4097, 129, 2), (977, 1, 5)])
def test_forms_with_unaligned_frames(bpc, lo, hi, w, h, nframes):
    """Odd frame sizes: frames start inside 16-byte vectors, chunk 0 takes the
    head and tail samples and the last chunk of a frame is partial, beside
    whole chunks that take the group forms."""
    ref, dist = synth.uniform_planes(w, h, nframes, 16, seed=900 + w + bpc, lo=lo, hi=hi)
    noise, moments = device_sums(ref, dist, bpc, entry="workspace_ff", prefill=-1)
    check(ref, dist, bpc, noise, moments)


def test_bright_form_past_2_53():
    """A bright 3840x2160 frame whose second moments pass 2^53 units: the
    exact sums from the bright form, within the bound of the CPU's."""
    ref, dist = synth.uniform_planes(3840, 2160, 1, 16, seed=61, lo=49152, hi=65535)
    noise, moments = device_sums(ref, dist, 16, entry="workspace_ff", prefill=-1)
    _, o2 = check(ref, dist, 16, noise, moments)
    assert int(o2[0, 3]) >= 1 << 53
