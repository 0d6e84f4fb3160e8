"""The device running float sum against O4, bit for bit (marked gpu).

vqx_float_running_sums_ws must return, for every buffer, the float the
psnr_hvs CPU extractor's accumulator holds after adding the buffer's terms
one by one ("ADR-1397: GPU psnr_hvs twins reproduce the CPU's running float
sum bit for bit", Context and Decision).  The buffers span several 4096-term
tiles with ragged ends, psnr_hvs-like term buffers up to the 3840x2160 count
(10 802 176 terms), sums that cross many binades, ties, subnormals, sums that
stall, overflow to infinity, and a sum the kernels' binade prediction gets
wrong on purpose.
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


def device_sums(terms: np.ndarray, prefill_workspace: bool = True) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(terms, dtype=np.float32)).cuda()
    if t.dim() == 1:
        t = t.unsqueeze(0)
    nb, n = t.shape
    ws = torch.full((max(vqx.float_sum_workspace_bytes(n, nb), 16),), 0xFF if prefill_workspace else 0,
                    dtype=torch.uint8, device="cuda:0")
    out = torch.full((nb,), -7.0, dtype=torch.float32, device="cuda:0")
    vqx.float_running_sums(t, out=out, workspace=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_bitwise(terms, got):
    want = oracle.running_float_sums(terms)
    gb, wb = got.view(np.uint32), want.view(np.uint32)
    bad = np.nonzero(gb != wb)[0]
    assert bad.size == 0, (f"{bad.size} of {gb.size} sums differ; first: buffer {int(bad[0])} "
                           f"device 0x{int(gb[bad[0]]):08x} oracle 0x{int(wb[bad[0]]):08x}")


@pytest.mark.parametrize("kind", ["uniform", "spread", "tiny", "ties", "stall", "ascending", "huge"])
@pytest.mark.parametrize("n", [1, 4095, 4096, 4097, 5 * 4096 + 123, 300_001])
def test_stress_buffers(kind, n):
    terms = synth.float_terms(n, kind, seed=40 + n % 97)
    assert_bitwise(terms[None, :], device_sums(terms))


@pytest.mark.parametrize("nblocks,nplanes,seed", [(1, 1, 1), (63, 3, 2), (1000, 4, 3), (20000, 2, 4)])
def test_hvs_like_buffers(nblocks, nplanes, seed):
    terms = synth.hvs_like_terms(nblocks, nplanes, seed=seed)
    assert_bitwise(terms, device_sums(terms))


def test_hvs_like_full_3840x2160_count():
    """Four planes of the 3840x2160 term count, 548 x 308 blocks of 64."""
    bw, bh = synth.HVS_4K_BLOCKS
    terms = synth.hvs_like_terms(bw * bh, 4, seed=1397)
    assert terms.shape[1] == 10_802_176
    assert_bitwise(terms, device_sums(terms))


def test_prediction_defeated():
    """The float sum stays at 2^24 - 1 while the exact total passes 2^24 a
    few terms in: every later term (0.49) rounds away, so the binade the
    kernels predict from the exact totals is never the sum's own."""
    n = 13 * 4096 + 17
    terms = np.full(n, 0.49, dtype=np.float32)
    terms[0] = np.float32(2 ** 24 - 1)
    got = device_sums(terms)
    assert float(got[0]) == 2 ** 24 - 1
    assert_bitwise(terms[None, :], got)


def test_many_buffers_one_call():
    """32 buffers of different content in one launch of each kernel."""
    rows = [synth.float_terms(20_000, k, seed=s) for s, k in
            enumerate(["uniform", "spread", "tiny", "ties", "stall", "ascending", "huge", "uniform"] * 4)]
    terms = np.stack(rows)
    assert_bitwise(terms, device_sums(terms))


def test_thousands_of_small_buffers():
    """4099 buffers of 700 terms in one call: the plan, map and walk grids
    far past the device's resident workgroups, each buffer one ragged tile."""
    kinds = ["uniform", "spread", "tiny", "ties", "stall", "ascending"]
    rows = [synth.float_terms(700, kinds[k % len(kinds)], seed=100 + k) for k in range(4099)]
    terms = np.stack(rows)
    assert_bitwise(terms, device_sums(terms))


def test_largest_buffer_count():
    """65535 buffers (the most a call takes) of 3 terms each."""
    rng = np.random.Generator(np.random.PCG64(65535))
    terms = (rng.random((65535, 3)) * 2.0 ** rng.integers(-20, 21, (65535, 3))).astype(np.float32)
    assert_bitwise(terms, device_sums(terms))


def test_zeros_and_edges():
    cases = [
        np.zeros(10_000, dtype=np.float32),
        np.full(9_000, -0.0, dtype=np.float32),
        np.array([2.0 ** -149] * 5000, dtype=np.float32),
        np.array([3.4028234663852886e38, 2.0 ** 103] + [0.0] * 5000, dtype=np.float32),
        np.ones(1 << 17, dtype=np.float32),
    ]
    for terms in cases:
        got = device_sums(terms)
        assert_bitwise(terms[None, :], got)
        assert np.signbit(got[0]) == np.signbit(oracle.running_float_sums(terms[None, :])[0])


def test_invalid_terms_give_nan_in_their_buffer_only():
    good = synth.float_terms(9000, "uniform", seed=1)
    rows = [good.copy() for _ in range(4)]
    rows[1][4321] = np.float32(-1.0)
    rows[2][8999] = np.float32(np.inf)
    rows[3][0] = np.float32(np.nan)
    got = device_sums(np.stack(rows))
    assert got.view(np.uint32)[0] == oracle.running_float_sums(good[None, :]).view(np.uint32)[0]
    for k in (1, 2, 3):
        assert got.view(np.uint32)[k] == 0x7FC00000, f"buffer {k}"


def test_no_terms_and_workspace_reuse():
    """nterms = 0 gives +0; one workspace serves calls of different sizes."""
    t = torch.zeros((3, 0), dtype=torch.float32, device="cuda:0")
    out = vqx.float_running_sums(t)
    torch.cuda.synchronize()
    assert out.cpu().numpy().view(np.uint32).tolist() == [0, 0, 0]
    big = synth.hvs_like_terms(3000, 2, seed=9)
    ws = torch.full((vqx.float_sum_workspace_bytes(big.shape[1], 2),), 0xFF, dtype=torch.uint8, device="cuda:0")
    for terms in (big, big[:, :5000].copy(), synth.float_terms(70_001, "ties", seed=3)[None, :], big):
        t = torch.from_numpy(np.ascontiguousarray(terms)).cuda()
        out = vqx.float_running_sums(t, workspace=ws)
        torch.cuda.synchronize()
        assert_bitwise(terms, out.cpu().numpy())


def test_calls_from_two_host_threads():
    """Calls on two streams from two host threads at once: each call's walk
    runs on the device's second stream, which the calls share in turn."""
    import threading
    inputs = [synth.hvs_like_terms(2500, 3, seed=20 + k) for k in range(2)]
    want = [oracle.running_float_sums(x) for x in inputs]
    errors = []

    def work(k):
        try:
            s = torch.cuda.Stream()
            t = torch.from_numpy(inputs[k]).cuda()
            torch.cuda.synchronize()
            for _ in range(6):
                with torch.cuda.stream(s):
                    out = vqx.float_running_sums(t, stream=s)
                s.synchronize()
                got = out.cpu().numpy()
                if not np.array_equal(got.view(np.uint32), want[k].view(np.uint32)):
                    errors.append((k, got, want[k]))
        except Exception as e:  # reported below, in the test's thread
            errors.append((k, repr(e)))

    threads = [threading.Thread(target=work, args=(k,)) for k in range(2)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[:2]


def test_graph_capture_replays():
    """The call captured into a graph (its second stream joins the capture)
    gives the eager result on every replay, with eager work between."""
    terms = synth.hvs_like_terms(1800, 2, seed=31)
    want = oracle.running_float_sums(terms)
    t = torch.from_numpy(terms).cuda()
    ws = torch.empty(vqx.float_sum_workspace_bytes(terms.shape[1], 2), dtype=torch.uint8, device="cuda:0")
    out = torch.full((2,), -7.0, dtype=torch.float32, device="cuda:0")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        vqx.float_running_sums(t, stream=s, out=out, workspace=ws)  # eager, before the capture
    s.synchronize()
    assert np.array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        vqx.float_running_sums(t, stream=s, out=out, workspace=ws)
    for k in range(3):
        out.fill_(-7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), (k, got, want)
        _ = (t * 2.0).sum().item()  # eager work between replays


def test_walk_beside_the_maps_gives_up(monkeypatch):
    """With the bound of one wait set to 0 the walk beside the map kernel
    gives up at its first wait; the walk after the map kernel (with its own
    takers of the queue) then walks those buffers, to the same bits."""
    monkeypatch.setenv("VQX_FLOAT_SUM_WAIT_TICKS", "0")
    cases = [synth.hvs_like_terms(2200, 3, seed=41),
             np.stack([synth.float_terms(3 * 4096 + 77, "ties", seed=5),
                       synth.float_terms(3 * 4096 + 77, "spread", seed=6)])]
    for terms in cases:
        assert_bitwise(terms, device_sums(terms))


def test_alternating_workspaces_and_inputs():
    """Calls alternate two workspaces and two inputs of different shapes: a
    record word left in a workspace by the call before last is never taken
    for this call's (every word is cleared before the maps are made)."""
    a = synth.hvs_like_terms(2600, 3, seed=51)
    b = np.stack([synth.float_terms(5 * 4096 + 9, kind, seed=52 + i) for i, kind in enumerate(("ties", "spread", "uniform"))])
    want = {0: oracle.running_float_sums(a), 1: oracle.running_float_sums(b)}
    ts = {0: torch.from_numpy(a).cuda(), 1: torch.from_numpy(b).cuda()}
    wss = [torch.full((max(vqx.float_sum_workspace_bytes(x.shape[1], 3) for x in (a, b)),), 0xFF,
                      dtype=torch.uint8, device="cuda:0") for _ in range(2)]
    for call in range(8):
        which = (call // 2) % 2  # inputs a, a, b, b, a, a, b, b; workspaces 0, 1, 0, 1, ...
        out = vqx.float_running_sums(ts[which], workspace=wss[call % 2])
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), want[which].view(np.uint32)), (call, got, want[which])


def test_walks_racing_for_buffers(monkeypatch):
    """A bound of 50 ticks (0.5 us): the walk after the map kernel claims
    most buffers while the walk beside it is still on them; the
    compare-and-swap on each buffer's done word lets exactly one write it."""
    monkeypatch.setenv("VQX_FLOAT_SUM_WAIT_TICKS", "50")
    terms = synth.hvs_like_terms(3000, 8, seed=61)
    for _ in range(3):
        assert_bitwise(terms, device_sums(terms))
