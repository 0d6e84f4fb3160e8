"""vqx_plane_stats_batch_noalloc against vqx_plane_stats_batch_ws (marked gpu).

The entry point for callers that cannot allocate keeps its scratch in one
fixed array per GPU.  Called through the C ABI twice in a row -- a large
batch, then a smaller one on another stream, over the scratch the first
left behind -- it must give the workspace form's sums bit for bit, and those
must be the exact integers of the oracle.  A batch beyond the array's size
is rejected before anything is queued.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from exact_reductions_amd import vqx  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vqx.lib()  # raises if libvqx.so is missing: no fallback exists


def _upload(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if a.dtype == np.uint16 else a.dtype)).cuda()


def _noalloc(ref, dist, bpc, stream):
    """The new entry point through the C ABI; host int64 noise [F], moments [F][4]."""
    f, h, w = ref.shape
    r, d = _upload(ref), _upload(dist)
    noise = torch.full((f,), -1, dtype=torch.int64, device="cuda:0")
    moments = torch.full((f, 4), -1, dtype=torch.int64, device="cuda:0")
    handle = stream.cuda_stream if stream is not None else None
    rc = vqx.lib().vqx_plane_stats_batch_noalloc(r.data_ptr(), d.data_ptr(), w, h, bpc, f, noise.data_ptr(),
                                                moments.data_ptr(), handle)
    assert rc == 0, vqx.status_string(rc)
    if stream is not None:
        stream.synchronize()
    torch.cuda.synchronize()
    return noise.cpu().numpy(), moments.cpu().numpy()


def _with_workspace(ref, dist, bpc):
    """The existing entry point with a caller workspace (0xFF-filled)."""
    f, h, w = ref.shape
    r, d = _upload(ref), _upload(dist)
    noise = torch.full((f,), -1, dtype=torch.int64, device="cuda:0")
    moments = torch.full((f, 4), -1, dtype=torch.int64, device="cuda:0")
    ws = torch.full((vqx.plane_stats_workspace_bytes(w, h, bpc, f),), 0xFF, dtype=torch.uint8, device="cuda:0")
    vqx.plane_stats_batch_ws(r, d, bpc, noise, moments, ws)
    torch.cuda.synchronize()
    return noise.cpu().numpy(), moments.cpu().numpy()


def test_two_calls_in_a_row_match_the_workspace_form():
    # first: the 3840x2160 16-bit workload, 32 frames (~1 MB of scratch)
    wl = synth.WORKLOADS[5]
    ref, dist = synth.generate(5)
    assert vqx.plane_stats_workspace_bytes(wl.w, wl.h, wl.bpc, wl.nframes) <= vqx.NOALLOC_SCRATCH_BYTES
    got = _noalloc(ref, dist, wl.bpc, None)
    want = _with_workspace(ref, dist, wl.bpc)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    exact = oracle.exact_batch_sums(ref[:4], dist[:4])
    assert np.array_equal(got[0][:4], exact[:, 0]) and np.array_equal(got[1][:4], exact[:, 1:])
    del ref, dist
    # second, smaller, on another stream, over the scratch the first left:
    # odd frames that start inside 16-byte vectors, at 12 bits
    ref, dist = synth.uniform_planes(1031, 577, 3, 16, seed=77, lo=0, hi=4095)
    side = torch.cuda.Stream()
    got = _noalloc(ref, dist, 12, side)
    want = _with_workspace(ref, dist, 12)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])
    exact = oracle.exact_batch_sums(ref, dist)
    assert np.array_equal(got[0], exact[:, 0]) and np.array_equal(got[1], exact[:, 1:])


def test_batch_beyond_the_scratch_is_rejected():
    """3840x2160 at 16 bits needs 507 records of 64 bytes per frame: 130
    frames need more than 4 MiB.  Nothing is queued and the outputs stay."""
    w, h, f = 3840, 2160, 130
    assert vqx.plane_stats_workspace_bytes(w, h, 16, f) > vqx.NOALLOC_SCRATCH_BYTES
    planes = torch.zeros(64, dtype=torch.int16, device="cuda:0")  # never read: rejected first
    noise = torch.full((f,), -1, dtype=torch.int64, device="cuda:0")
    moments = torch.full((f, 4), -1, dtype=torch.int64, device="cuda:0")
    rc = vqx.lib().vqx_plane_stats_batch_noalloc(planes.data_ptr(), planes.data_ptr(), w, h, 16, f,
                                                noise.data_ptr(), moments.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == vqx.E_SCRATCH
    assert bool((noise == -1).all()) and bool((moments == -1).all())
