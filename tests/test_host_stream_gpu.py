"""Host-fed batches on the device (marked gpu).

``vqx_plane_stats_host_ws`` uploads a batch from host memory in sub-batches
while reducing the ones before; its sums must equal the exact oracle (O2)
and the device-resident entry point, element by element, for every upload
size (including a last, smaller upload), pinned and pageable host memory,
the library's own copy stream, a caller's and the compute stream itself.
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
    vqx.lib()


def check(ref, dist, bpc, fpu, pinned=True, copy_stream=None, label=""):
    if pinned:
        r = torch.from_numpy(ref).pin_memory()
        d = torch.from_numpy(dist).pin_memory()
    else:
        r, d = ref, dist
    noise, moments = vqx.plane_stats_host(r, d, bpc, frames_per_upload=fpu, copy_stream=copy_stream)
    noise, moments = noise.cpu().numpy(), moments.cpu().numpy()
    want = oracle.exact_batch_sums(ref, dist)
    got = np.concatenate([noise[:, None], moments], 1)
    assert (got == want).all(), label
    # the same as the device-resident entry point
    n2, m2 = vqx.plane_stats_batch(torch.from_numpy(ref).cuda(), torch.from_numpy(dist).cuda(), bpc)
    torch.cuda.synchronize()
    assert (n2.cpu().numpy() == noise).all() and (m2.cpu().numpy() == moments).all()


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("fpu", [1, 3, 64])
def test_workloads(n, fpu):
    wl = synth.WORKLOADS[n]
    ref, dist = synth.generate(n, nframes=min(wl.nframes, 7))
    check(ref, dist, wl.bpc, fpu, label=f"workload {n}, {fpu} per upload")


def test_pageable_host_memory():
    ref, dist = synth.generate(2, nframes=5)
    check(ref, dist, 10, 2, pinned=False)


def test_caller_copy_stream_and_one_stream():
    ref, dist = synth.generate(4, nframes=6)
    side = torch.cuda.Stream()  # default priority
    check(ref, dist, 16, 2, copy_stream=side, label="caller's copy stream")
    check(ref, dist, 16, 2, copy_stream=torch.cuda.current_stream(), label="one stream")


@pytest.mark.parametrize("w,h,f,bpc,fpu", [(17, 9, 7, 8, 2), (1, 1, 5, 16, 3), (4097, 3, 4, 16, 3),
                                           (962, 541, 9, 12, 4)])
def test_odd_shapes(w, h, f, bpc, fpu):
    """Frames that do not start on a 16-byte boundary inside an upload."""
    ref, dist = synth.uniform_planes(w, h, f, bpc, seed=w + h, container_max=True)
    check(ref, dist, bpc, fpu, label=f"{w}x{h}x{f}")


def test_outputs_written_not_accumulated():
    ref, dist = synth.generate(1, nframes=4)
    f, h, w = ref.shape
    L = vqx.lib()
    out = torch.full((5 * f,), -1, dtype=torch.int64, device="cuda")
    ws = torch.full((vqx.plane_stats_host_workspace_bytes(w, h, 8, 3),), 0xFF, dtype=torch.uint8, device="cuda")
    r = torch.from_numpy(ref).pin_memory()
    d = torch.from_numpy(dist).pin_memory()
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert L.vqx_plane_stats_host_ws(r.data_ptr(), d.data_ptr(), w, h, 8, f, 3, out[:f].data_ptr(),
                                         out[f:].data_ptr(), ws.data_ptr(), ws.numel(), st, None) == 0
    o = out.cpu().numpy()
    want = oracle.exact_batch_sums(ref, dist)
    assert (np.concatenate([o[:f, None], o[f:].reshape(f, 4)], 1) == want).all()
