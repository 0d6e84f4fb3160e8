"""The entry points captured into a HIP graph and replayed (marked gpu).

A caller may capture a call into a graph and replay it many times (a
serving loop, say).  Each captured call below is replayed three times, with
the program's own eager work and synchronisations between the replays, and
with the input planes rewritten in place between some replays: every replay
must give what an eager call gives on the planes as they are then, and the
exact sums must be the oracle's.  None of the library's launches records a
memset: outputs are written, never cleared and added to.
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


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16 if a.dtype == np.uint16 else a.dtype)).cuda()


def _replay_against_eager(call, inputs, contents, eager):
    """Capture call() on a side stream, then for each content set: copy it
    into the input tensors in place, replay, and compare the outputs with
    eager(content)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(s)  # once eagerly: the library's one-time set-up happens outside the capture
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        outs = call(s)
    for k, content in enumerate(contents):
        for t, a in zip(inputs, content):
            t.copy_(_dev(a))
        for o in outs:
            o.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [o.cpu().numpy().copy() for o in outs]
        want = eager(content)
        for i, (x, y) in enumerate(zip(got, want)):
            assert np.array_equal(x, y), f"replay {k}, output {i}"
        _ = (inputs[0].float() * 2.0).sum().item()  # eager work between replays


def _uniform16(seed, f, h, w, lo, hi):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.integers(lo, hi, size=(f, h, w), endpoint=True).astype(np.uint16),
            rng.integers(lo, hi, size=(f, h, w), endpoint=True).astype(np.uint16))


def test_exact_sums_workspace_form():
    f, h, w = 3, 717, 1031
    cases = [_uniform16(1, f, h, w, 0, 65535), _uniform16(2, f, h, w, 49152, 65535), _uniform16(3, f, h, w, 0, 4095)]
    R, D = _dev(cases[0][0]), _dev(cases[0][1])
    noise = torch.empty(f, dtype=torch.int64, device="cuda:0")
    moments = torch.empty((f, 4), dtype=torch.int64, device="cuda:0")
    ws = torch.empty(vqx.plane_stats_workspace_bytes(w, h, 16, f), dtype=torch.uint8, device="cuda:0")

    def call(s):
        vqx.plane_stats_batch_ws(R, D, 16, noise, moments, ws, stream=s)
        return [noise, moments]

    def eager(content):
        o2 = oracle.exact_batch_sums(*content)
        return [o2[:, 0], o2[:, 1:]]

    _replay_against_eager(call, [R, D], cases, eager)


def test_exact_sums_allocation_free_form():
    """The entry point for callers that cannot allocate, in a graph: its
    fixed scratch keeps the last replay's records, and each replay writes
    its own over them."""
    wl = synth.WORKLOADS[4]
    ref, dist = synth.generate(4, nframes=6)
    other = _uniform16(4, *ref.shape, 56000, 64000)
    R, D = _dev(ref), _dev(dist)
    f = ref.shape[0]
    noise = torch.empty(f, dtype=torch.int64, device="cuda:0")
    moments = torch.empty((f, 4), dtype=torch.int64, device="cuda:0")

    def call(s):
        vqx.plane_stats_batch_noalloc(R, D, wl.bpc, noise, moments, stream=s)
        return [noise, moments]

    def eager(content):
        o2 = oracle.exact_batch_sums(*content)
        return [o2[:, 0], o2[:, 1:]]

    _replay_against_eager(call, [R, D], [(ref, dist), other, (ref, dist)], eager)


def test_cpu_order_form_past53():
    """The CPU-order form (stage 1, maps, walk) on a frame past 2^53 whose
    adds round, then on bright content whose sums need no walk."""
    ref, dist = synth.past53_mixed()
    bright = _uniform16(5, *ref.shape, 57344, 65535)
    f, h, w = ref.shape
    R, D = _dev(ref), _dev(dist)
    out = torch.empty((2, 5 * f), dtype=torch.int64, device="cuda:0")
    ws = torch.empty(vqx.plane_stats_cpu_order_workspace_bytes(w, h, 16, f), dtype=torch.uint8, device="cuda:0")

    def call(s):
        assert vqx.lib().vqx_plane_stats_batch_cpu_order_ws(
            R.data_ptr(), D.data_ptr(), w, h, 16, f, out[0, :f].data_ptr(), out[0, f:].data_ptr(),
            out[1, :f].data_ptr(), out[1, f:].data_ptr(), ws.data_ptr(), ws.numel(), s.cuda_stream) == 0
        return [out]

    def eager(content):
        r, d = content
        o2 = oracle.exact_batch_sums(r, d)
        o1 = oracle.seq_batch_sums(r, d, 16)
        exact = np.concatenate([o2[:, 0], o2[:, 1:].reshape(-1)])
        cpu = np.array([[int(float(o1[i][k]) * float(256 ** p)) for k, p in enumerate(oracle.UNIT_POWER)]
                        for i in range(f)], dtype=np.int64)
        return [np.stack([exact, np.concatenate([cpu[:, 0], cpu[:, 1:].reshape(-1)])])]

    _replay_against_eager(call, [R, D], [(ref, dist), bright, (ref, dist)], eager)


def test_integer_psnr_of_views():
    """The integer psnr twin over pitched regions (the view kernels)."""
    rng = np.random.Generator(np.random.PCG64(6))
    f, H, W = 2, 300, 1000
    big = [rng.integers(0, 1023, size=(f, H, W), endpoint=True).astype(np.uint16) for _ in range(4)]
    sl = (slice(None), slice(7, 290), slice(5, 941))
    BR, BD = _dev(big[0]), _dev(big[1])
    R, D = BR[sl], BD[sl]
    ws = torch.empty(vqx.plane_view_workspace_bytes(936, 283, 10, f), dtype=torch.uint8, device="cuda:0")
    noise = torch.empty(f, dtype=torch.int64, device="cuda:0")
    _, args = vqx._views(R, D, 10)

    def call(s):
        assert vqx.lib().vqx_psnr_int_view_ws(*args, 936, 283, 10, f, noise.data_ptr(), ws.data_ptr(), ws.numel(),
                                              s.cuda_stream) == 0
        return [noise]

    def eager(content):
        r, d = content
        return [np.array([oracle.int_noise(r[i][sl[1:]], d[i][sl[1:]]) for i in range(f)], dtype=np.int64)]

    _replay_against_eager(call, [BR, BD], [(big[0], big[1]), (big[2], big[3])], eager)
