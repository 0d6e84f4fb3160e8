"""The CPU's running double sums, reproduced on the device (marked gpu).

``vqx_plane_stats_batch_cpu_order_ws`` returns, besides the exact sums, the
value each of the CPU extractor's double accumulators holds after its last
add.  The oracle's sequential C loop (``oracle.seq_batch_sums``) is that
accumulator itself, so the check is plain bitwise equality on every frame
and output -- past 2^53 too, where the exact sums only meet the bound.
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


UNIT_POWER = (2, 1, 1, 2, 2)


def run(ref, dist, bpc):
    r = torch.from_numpy(np.ascontiguousarray(ref)).to("cuda:0")
    d = torch.from_numpy(np.ascontiguousarray(dist)).to("cuda:0")
    n, m, cn, cm = vqx.plane_stats_batch_cpu_order(r, d, bpc)
    torch.cuda.synchronize()
    return n.cpu().numpy(), m.cpu().numpy(), cn.cpu().numpy(), cm.cpu().numpy()


def check(ref, dist, bpc, expect_past53=None):
    """Exact sums equal the exact oracle; CPU-order sums equal the CPU's
    sequential doubles bit for bit; their conclusions equal the CPU's."""
    h, w = ref.shape[1:]
    n, m, cn, cm = run(ref, dist, bpc)
    o1 = oracle.seq_batch_sums(ref, dist, bpc)
    o2 = oracle.exact_batch_sums(ref, dist)
    s = 1 << (bpc - 8)
    past = 0
    for f in range(ref.shape[0]):
        exact = [int(n[f])] + [int(v) for v in m[f]]
        cpu = [int(cn[f])] + [int(v) for v in cm[f]]
        assert exact == [int(v) for v in o2[f]], f"frame {f}: exact sums"
        for k in range(5):
            want = float(o1[f][k]) * float(s ** UNIT_POWER[k])
            assert float(cpu[k]) == want and cpu[k] == int(want), (
                f"frame {f} output {k}: device {cpu[k]} CPU {int(want)} exact {exact[k]}")
            if exact[k] >= oracle.TWO53:
                past += 1
        concl = vqx.conclude_batch([cpu[0]], [cpu[1:]], w, h, bpc)[0]
        want_concl = oracle.conclude_from_doubles(o1[f], w, h)
        assert [concl[0]] + list(concl[2:]) == list(want_concl), f"frame {f}: conclusion"
    if expect_past53 is not None:
        assert (past > 0) == expect_past53
    return past


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_workloads(n):
    wl = synth.WORKLOADS[n]
    ref, dist = synth.generate(n, nframes=min(wl.nframes, 8))
    check(ref, dist, wl.bpc, expect_past53=(n == 5))


def test_past53_mixed_bit_identical():
    """The 2560x1440 frame in which one sample in ten is below 4096: the CPU's
    adds round, and the device returns the CPU's rounded value exactly."""
    ref, dist = synth.past53_mixed(nframes=2)
    assert check(ref, dist, 16, expect_past53=True) == 4


def test_past53_full_range_bit_identical():
    ref, dist = synth.past53_fullrange(nframes=2)
    check(ref, dist, 16, expect_past53=True)


def test_odd_dark_samples_past54():
    """Odd dark squares among bright ones: they tie at 2^53..2^54 (one unit
    of rounding there) but not past 2^54, where runs holding them round
    without ties -- a case between the runs whose terms all are multiples of
    the binade's unit and those with ties."""
    ref, dist = synth.odd_dark_bright()
    h, w = ref.shape[1:]
    assert oracle.exact_frame_sums(ref[0], dist[0])[3] >= 2 * oracle.TWO53
    check(ref, dist, 16, expect_past53=True)


def _mid_bright(w, h, seed):
    """A tenth of the samples in 4096..5792 (float squares in [2^24, 2^25):
    multiples of 4 -- an odd square ties at 25 bits and goes to the even
    significand -- some 4 mod 8), the rest in 49152..65535 (float squares
    multiples of 2^8); both planes drawn alike."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(2):
        low = rng.random(size=(1, h, w)) < 0.1
        mid = rng.integers(4096, 5792, size=(1, h, w), endpoint=True, dtype=np.uint16)
        bright = rng.integers(49152, 65535, size=(1, h, w), endpoint=True, dtype=np.uint16)
        out.append(np.where(low, mid, bright).astype(np.uint16))
    return out[0], out[1]


@pytest.mark.parametrize("w,h,walked", [(2560, 1440, False), (3840, 2160, False), (8192, 4096, True)])
def test_shared_trailing_zeros_past53(w, h, walked):
    """Terms that all are multiples of 2^j keep every partial sum a multiple
    of 2^j, which a double holds exactly below 2^(53+j): there the CPU's sum
    is the exact one, past 2^53 or not.  Here j = 2 for the squares of ref
    and dist.  At 2560x1440 they end between 2^53 and 2^54, at 3840x2160
    between 2^54 and 2^55 (no add rounds); in the largest frame, 2^25
    samples, past 2^55, where the terms that are 4 mod 8 tie and the CPU's
    sum rounds."""
    ref, dist = _mid_bright(w, h, seed=w + h)
    for plane in (ref, dist):
        sq = plane.astype(np.float32) * plane.astype(np.float32)  # binary32 squares, as the CPU's
        terms = sq.astype(np.uint64)
        low = int(np.bitwise_or.reduce(terms.ravel() & np.uint64(15)))
        assert (low & -low) == 4  # j = 2
        total = int(terms.sum(dtype=np.uint64))
        assert oracle.TWO53 <= total and (total >= 4 * oracle.TWO53) == walked
    o1 = oracle.seq_batch_sums(ref, dist, 16)
    o2 = oracle.exact_batch_sums(ref, dist)
    for k in (3, 4):
        cpu = float(o1[0][k]) * float(256 ** UNIT_POWER[k])  # in the integer units of the exact sum
        assert (int(cpu) != int(o2[0][k])) == walked  # the CPU rounds past 2^(53+j) only
    check(ref, dist, 16, expect_past53=True)


def test_container_values_above_bpc():
    """A 10-bit container holding full-range values passes 2^53 too."""
    ref, dist = synth.uniform_planes(3840, 2160, 1, 10, seed=11, container_max=True)
    check(ref, dist, 10, expect_past53=True)


@pytest.mark.parametrize("bpc", [13, 14, 15])
def test_depths_13_to_15(bpc):
    ref, dist = synth.uniform_planes(3840, 2160, 1, bpc, seed=bpc, container_max=True)
    check(ref, dist, bpc, expect_past53=True)


def test_unaligned_frame_starts_past53():
    """Odd frame sizes: frames 1 and 2 start inside a 16-byte vector, so the
    head and tail samples of each frame are walked separately, first and
    last, in the CPU's order."""
    ref, dist = synth.uniform_planes(4097, 2049, 3, 16, seed=4097, container_max=True)
    check(ref, dist, 16, expect_past53=True)


def test_empty_last_chunk_past53():
    """3779x1305 = 8*(2048*301 + 1) + 3 samples: frame 0 has 2048*301 + 1
    whole vectors, so a frame takes 302 chunks, but frame 1 starts 3 samples
    past a vector boundary and has one vector fewer -- its last chunk is
    empty, after the sums have passed 2^53 (and 2^54)."""
    w, h = 3779, 1305
    assert w * h == 8 * (2048 * 301 + 1) + 3
    ref, dist = synth.uniform_planes(w, h, 3, 16, seed=3779, lo=60000, hi=65535)
    assert check(ref, dist, 16, expect_past53=True) == 6


def test_largest_frame_past53():
    """2^25 samples at full range: the sums reach binade 55."""
    ref, dist = synth.uniform_planes(8192, 4096, 1, 16, seed=25, container_max=True)
    check(ref, dist, 16, expect_past53=True)


def test_constant_worst_case():
    """65535 against 0 everywhere: every noise term is 4294836224 and the
    noise passes 2^54; all rounding steps meet the same term."""
    ref, dist = synth.constant_pair(3840, 2160, 1, 16, 65535, 0)
    check(ref, dist, 16, expect_past53=True)


def test_ties_past53():
    """Terms that are odd multiples of half an ulp: with u = 2 (binade 53)
    every odd term is a tie, decided by the sum's parity."""
    rng = np.random.Generator(np.random.PCG64(53))
    ref = rng.integers(46341, 65535, size=(1, 2160, 3840), endpoint=True).astype(np.uint16)
    ref[:, ::2] = rng.integers(1, 4095, size=(1, 1080, 3840)).astype(np.uint16) | 1
    dist = np.zeros_like(ref)
    check(ref, dist, 16)


def test_small_frames_equal_exact():
    ref, dist = synth.uniform_planes(18, 22, 50, 16, seed=3, container_max=True)
    check(ref, dist, 16, expect_past53=False)


def _check_outputs(ref, dist, bpc, out, f):
    o1 = oracle.seq_batch_sums(ref, dist, bpc)
    o2 = oracle.exact_batch_sums(ref, dist)
    s = 1 << (bpc - 8)
    o = out.cpu().numpy()
    for k in range(f):
        exact = [int(o[0, k])] + [int(v) for v in o[0, f + 4 * k:f + 4 * k + 4]]
        cpu = [int(o[1, k])] + [int(v) for v in o[1, f + 4 * k:f + 4 * k + 4]]
        assert exact == [int(v) for v in o2[k]], f"frame {k}: exact sums"
        for j in range(5):
            assert cpu[j] == int(float(o1[k][j]) * float(s ** UNIT_POWER[j])), f"frame {k} output {j}"


def test_reused_workspace_and_side_stream():
    """One workspace, filled with 0xFF first, serves batches of different
    content, depth and size in turn on a non-default stream: nothing a call
    reads is left over from an earlier call (the queue lengths, chunk
    cases and maps are all written afresh), and outputs are written, not
    added to."""
    mixed = synth.past53_mixed(nframes=2)
    odd = synth.odd_dark_bright(w=2560, h=1440, nframes=2)
    small8 = synth.uniform_planes(333, 77, 4, 8, seed=8)
    batches = [(mixed, 16), (odd, 16), (small8, 8), (mixed, 16)]
    need = max(vqx.plane_stats_cpu_order_workspace_bytes(r.shape[2], r.shape[1], b, r.shape[0])
               for (r, _), b in batches)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda:0")
    side = torch.cuda.Stream()
    L = vqx.lib()
    for (ref, dist), bpc in batches:
        f, h, w = ref.shape
        r = torch.from_numpy(ref).cuda()
        d = torch.from_numpy(dist).cuda()
        out = torch.full((2, 5 * f), -1, dtype=torch.int64, device="cuda:0")
        torch.cuda.synchronize()
        with torch.cuda.stream(side):
            assert L.vqx_plane_stats_batch_cpu_order_ws(
                r.data_ptr(), d.data_ptr(), w, h, bpc, f, out[0, :f].data_ptr(), out[0, f:].data_ptr(),
                out[1, :f].data_ptr(), out[1, f:].data_ptr(), ws.data_ptr(), need, side.cuda_stream) == 0
        side.synchronize()
        _check_outputs(ref, dist, bpc, out, f)


def _view_case(ref_np, dist_np, R, D, bpc):
    """The view form against the sequential oracle on the selected samples,
    and against the contiguous form."""
    n, m, cn, cm = vqx.plane_stats_view_cpu_order(R, D, bpc)
    torch.cuda.synchronize()
    f = ref_np.shape[0]
    out = torch.stack([torch.cat([n, m.reshape(-1)]), torch.cat([cn, cm.reshape(-1)])])
    ref_c, dist_c = np.ascontiguousarray(ref_np), np.ascontiguousarray(dist_np)
    _check_outputs(ref_c, dist_c, bpc, out, f)
    n2, m2, cn2, cm2 = run(ref_c, dist_c, bpc)
    assert (n.cpu().numpy() == n2).all() and (cn.cpu().numpy() == cn2).all()
    assert (m.cpu().numpy() == m2).all() and (cm.cpu().numpy() == cm2).all()


def test_view_form_pitched_region_past53():
    """A 2560x1440 region of padded 16-bit planes whose sums pass 2^53."""
    ref, dist = synth.past53_mixed(nframes=2)
    f, h, w = ref.shape
    big_r = np.zeros((f, h + 3, w + 70), dtype=np.uint16)
    big_d = np.zeros_like(big_r)
    big_r[:, 2:2 + h, 5:5 + w] = ref
    big_d[:, 2:2 + h, 5:5 + w] = dist
    sl = (slice(None), slice(2, 2 + h), slice(5, 5 + w))
    R, D = torch.from_numpy(big_r).cuda()[sl], torch.from_numpy(big_d).cuda()[sl]
    _view_case(big_r[sl], big_d[sl], R, D, 16)


@pytest.mark.parametrize("bpc", [8, 12, 16])
def test_view_form_odd_layouts(bpc):
    """Odd pitches, ref and dist at different offsets, frame stride 0."""
    rng = np.random.default_rng(bpc)
    hi = 255 if bpc == 8 else 65535
    dt = np.uint8 if bpc == 8 else np.uint16
    big_r = rng.integers(0, hi, size=(3, 41, 101), endpoint=True).astype(dt)
    big_d = rng.integers(0, hi, size=(3, 43, 97), endpoint=True).astype(dt)
    R = torch.from_numpy(big_r).cuda()[:, 1:40, 3:90]
    D = torch.from_numpy(big_d).cuda()[:, 2:41, 0:87]
    _view_case(big_r[:, 1:40, 3:90], big_d[:, 2:41, 0:87], R, D, bpc)
    one_r = torch.from_numpy(big_r[:1]).cuda().expand(4, 41, 101)
    one_d = torch.from_numpy(big_d[:1, :41, :97]).cuda().expand(4, 41, 97)[:, :, :97]
    _view_case(np.broadcast_to(big_r[:1, :, :97], (4, 41, 97)), np.broadcast_to(big_d[:1, :41, :97], (4, 41, 97)),
               one_r[:, :, :97], one_d, bpc)


def _in_place_case(ref_np, dist_np, R, D, bpc, in_place=True):
    """The view form through the C ABI with a workspace filled with 0xA5:
    results as in _view_case, and views whose rows are whole vectors read
    in place (the part of the workspace past the contiguous form's is
    left as it was), others gathered into it."""
    f, h, w = R.shape
    total = vqx.plane_stats_view_cpu_order_workspace_bytes(w, h, bpc, f)
    own = vqx.plane_stats_cpu_order_workspace_bytes(w, h, bpc, f)
    ws = torch.full((total,), 0xA5, dtype=torch.uint8, device="cuda:0")
    out = torch.full((2, 5 * f), -1, dtype=torch.int64, device="cuda:0")
    _, args = vqx._views(R, D, bpc)
    torch.cuda.synchronize()
    assert vqx.lib().vqx_plane_stats_view_cpu_order_ws(
        *args, w, h, bpc, f, out[0, :f].data_ptr(), out[0, f:].data_ptr(), out[1, :f].data_ptr(),
        out[1, f:].data_ptr(), ws.data_ptr(), total, torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    untouched = bool((ws[own:] == 0xA5).all())
    assert untouched == in_place, "read in place" if in_place else "gathered"
    _check_outputs(np.ascontiguousarray(ref_np), np.ascontiguousarray(dist_np), bpc, out, f)
    n2, m2, cn2, cm2 = run(np.ascontiguousarray(ref_np), np.ascontiguousarray(dist_np), bpc)
    o = out.cpu().numpy()
    assert (o[0, :f] == n2).all() and (o[1, :f] == cn2).all()
    assert (o[0, f:] == m2.reshape(-1)).all() and (o[1, f:] == cm2.reshape(-1)).all()


def test_view_form_in_place_past53():
    """A 2560x1440 region, 8 samples in, of 16-bit planes with different
    pitches (2624 and 2696 samples), sums past 2^53: read in place."""
    ref, dist = synth.past53_mixed(nframes=2)
    f, h, w = ref.shape
    big_r = np.zeros((f, h + 3, w + 64), dtype=np.uint16)
    big_d = np.zeros((f, h + 4, w + 136), dtype=np.uint16)
    big_r[:, 2:2 + h, 8:8 + w] = ref
    big_d[:, 3:3 + h, 16:16 + w] = dist
    sr = (slice(None), slice(2, 2 + h), slice(8, 8 + w))
    sd = (slice(None), slice(3, 3 + h), slice(16, 16 + w))
    R, D = torch.from_numpy(big_r).cuda()[sr], torch.from_numpy(big_d).cuda()[sd]
    _in_place_case(big_r[sr], big_d[sd], R, D, 16)


def test_view_form_in_place_repeated_frame():
    """Frame stride 0 on both sides (one frame pair read three times) and a
    contiguous dist beside a pitched ref: read in place."""
    ref, dist = synth.odd_dark_bright(w=2560, h=1440, nframes=1)
    h, w = ref.shape[1:]
    big_r = np.zeros((1, h, w + 8), dtype=np.uint16)
    big_r[:, :, :w] = ref
    R = torch.from_numpy(big_r).cuda()[:, :, :w].expand(3, h, w)
    D = torch.from_numpy(dist).cuda().expand(3, h, w)
    _in_place_case(np.broadcast_to(ref, (3, h, w)), np.broadcast_to(dist, (3, h, w)), R, D, 16)


@pytest.mark.parametrize("bpc", [9, 12, 16])
@pytest.mark.parametrize("w,h,x0", [(8, 1, 0), (8, 300, 8), (96, 37, 16), (1024, 65, 8), (4096, 17, 24)])
def test_view_form_in_place_small(bpc, w, h, x0):
    """Small aligned views (rows of one vector, chunks with a ragged tail,
    rows longer than a chunk's share) at several depths: read in place."""
    rng = np.random.default_rng(w * 131 + h * 7 + bpc)
    hi = (1 << bpc) - 1
    big_r = rng.integers(0, hi, size=(3, h + 2, w + x0 + 40), endpoint=True).astype(np.uint16)
    big_d = rng.integers(0, hi, size=(3, h + 1, w + x0 + 8), endpoint=True).astype(np.uint16)
    sr = (slice(None), slice(1, 1 + h), slice(x0, x0 + w))
    sd = (slice(None), slice(0, h), slice(x0, x0 + w))
    R, D = torch.from_numpy(big_r).cuda()[sr], torch.from_numpy(big_d).cuda()[sd]
    _in_place_case(big_r[sr], big_d[sd], R, D, bpc)


def test_view_form_in_place_15bit_past53():
    """A 4096x4096 15-bit frame pair (bright, a few dark odd samples) inside
    planes with 64 samples of row padding: the squares' sums pass 2^53 units
    of 1/s^2, read in place."""
    rng = np.random.default_rng(1515)
    h = w = 4096
    planes = []
    for _ in range(2):
        x = rng.integers(28000, 32767, size=(1, h, w), endpoint=True)
        dark = rng.random((1, h, w)) < 0.02
        x = np.where(dark, rng.integers(0, 2047, size=(1, h, w), endpoint=True) | 1, x).astype(np.uint16)
        big = np.zeros((1, h, w + 64), dtype=np.uint16)
        big[:, :, 32:32 + w] = x
        planes.append(big)
    sl = (slice(None), slice(None), slice(32, 32 + w))
    o2 = oracle.exact_batch_sums(np.ascontiguousarray(planes[0][sl]), np.ascontiguousarray(planes[1][sl]))
    assert o2[0][3] >= 2**53 and o2[0][4] >= 2**53
    _in_place_case(planes[0][sl], planes[1][sl], torch.from_numpy(planes[0]).cuda()[sl],
                   torch.from_numpy(planes[1]).cuda()[sl], 15)


def test_view_form_unaligned_gathered():
    """A view 4 samples in with a pitch of 122 samples (its rows start at
    different offsets within 16 bytes): read in place; one of width 100
    (rows not whole vectors): gathered; same results."""
    rng = np.random.default_rng(7)
    big = rng.integers(0, 65535, size=(2, 50, 122), endpoint=True).astype(np.uint16)
    big_d = rng.integers(0, 65535, size=(2, 50, 122), endpoint=True).astype(np.uint16)
    s4 = (slice(None), slice(None), slice(4, 100))
    _in_place_case(big[s4], big_d[s4], torch.from_numpy(big).cuda()[s4], torch.from_numpy(big_d).cuda()[s4], 16)
    s100 = (slice(None), slice(None), slice(0, 100))
    _in_place_case(big[s100], big_d[s100], torch.from_numpy(big).cuda()[s100],
                   torch.from_numpy(big_d).cuda()[s100], 16, in_place=False)


@pytest.mark.parametrize("xr,xd", [(4, 4), (1, 7), (0, 3), (5, 0), (2, 6)])
def test_view_form_shifted_in_place(xr, xd):
    """Views xr and xd samples in (so 2*xr and 2*xd bytes into 16-byte
    blocks) of planes whose pitches are whole vectors: read in place, two
    blocks per vector, same results."""
    rng = np.random.default_rng(70 + 8 * xr + xd)
    big = rng.integers(0, 65535, size=(3, 50, 128), endpoint=True).astype(np.uint16)
    big_d = rng.integers(0, 65535, size=(3, 51, 136), endpoint=True).astype(np.uint16)
    sr = (slice(None), slice(None), slice(xr, xr + 96))
    sd = (slice(None), slice(1, 51), slice(xd, xd + 96))
    _in_place_case(big[sr], big_d[sd], torch.from_numpy(big).cuda()[sr], torch.from_numpy(big_d).cuda()[sd], 16)


@pytest.mark.parametrize("pr,pd,xr,xd", [(122, 122, 4, 4), (122, 122, 4, 5), (122, 131, 0, 0), (125, 127, 3, 1),
                                         (121, 129, 2, 2)])
def test_view_form_varying_phases_in_place(pr, pd, xr, xd):
    """Pitches that are not whole vectors: each row starts at its own offset
    within 16 bytes (the same in ref and dist, or not); read in place."""
    rng = np.random.default_rng(pr * 1000 + pd + 10 * xr + xd)
    big = rng.integers(0, 65535, size=(3, 40, pr), endpoint=True).astype(np.uint16)
    big_d = rng.integers(0, 65535, size=(3, 41, pd), endpoint=True).astype(np.uint16)
    sr = (slice(None), slice(None), slice(xr, xr + 96))
    sd = (slice(None), slice(1, 41), slice(xd, xd + 96))
    _in_place_case(big[sr], big_d[sd], torch.from_numpy(big).cuda()[sr], torch.from_numpy(big_d).cuda()[sd], 16)


@pytest.mark.parametrize("er,ed", [(61, 63), (60, 60)])
def test_view_form_varying_phases_in_place_past53(er, ed):
    """The 2560x1440 region past 2^53 in planes whose pitches are w + er and
    w + ed samples (rows at varying offsets within 16 bytes), 5 and 7
    samples in: the maps and the walk cut each vector from its row."""
    ref, dist = synth.past53_mixed(nframes=2)
    f, h, w = ref.shape
    big_r = np.zeros((f, h + 3, w + er), dtype=np.uint16)
    big_d = np.zeros((f, h + 4, w + ed), dtype=np.uint16)
    big_r[:, 2:2 + h, 5:5 + w] = ref
    big_d[:, 3:3 + h, 7:7 + w] = dist
    sr = (slice(None), slice(2, 2 + h), slice(5, 5 + w))
    sd = (slice(None), slice(3, 3 + h), slice(7, 7 + w))
    R, D = torch.from_numpy(big_r).cuda()[sr], torch.from_numpy(big_d).cuda()[sd]
    _in_place_case(big_r[sr], big_d[sd], R, D, 16)


@pytest.mark.parametrize("xr,xd", [(11, 21), (13, 13)])
def test_view_form_shifted_in_place_past53(xr, xd):
    """The 2560x1440 case past 2^53 with the regions 11 and 21 (and 13 and
    13) samples in: the maps and the walk read shifted vectors in place."""
    ref, dist = synth.past53_mixed(nframes=2)
    f, h, w = ref.shape
    big_r = np.zeros((f, h + 3, w + 64), dtype=np.uint16)
    big_d = np.zeros((f, h + 4, w + 136), dtype=np.uint16)
    big_r[:, 2:2 + h, xr:xr + w] = ref
    big_d[:, 3:3 + h, xd:xd + w] = dist
    sr = (slice(None), slice(2, 2 + h), slice(xr, xr + w))
    sd = (slice(None), slice(3, 3 + h), slice(xd, xd + w))
    R, D = torch.from_numpy(big_r).cuda()[sr], torch.from_numpy(big_d).cuda()[sd]
    _in_place_case(big_r[sr], big_d[sd], R, D, 16)


@pytest.mark.parametrize("seed", range(3))
def test_random_views_in_place_past53(seed):
    """Seeded random batches past 2^53 as in the contiguous tests, widths
    rounded to whole vectors, inside planes with random padded pitches."""
    rng = np.random.default_rng(40530 + seed)
    ref, dist, desc = _random_case(rng)
    f, h, w = ref.shape
    w8 = w - w % 8
    pads = [int(rng.integers(0, 9)) * 8 for _ in range(4)]
    views = []
    for plane, (x0, extra) in zip((ref, dist), ((pads[0], pads[1]), (pads[2], pads[3]))):
        big = np.zeros((f, h, x0 + w8 + extra), dtype=np.uint16)
        big[:, :, x0:x0 + w8] = plane[:, :, :w8]
        sl = (slice(None), slice(None), slice(x0, x0 + w8))
        views.append((big[sl], torch.from_numpy(big).cuda()[sl]))
    (rn, R), (dn, D) = views
    _in_place_case(rn, dn, R, D, 16)


@pytest.mark.parametrize("seed", range(2))
def test_random_views_shifted_in_place_past53(seed):
    """As above, the regions at any sample offset in rows of any pitch."""
    rng = np.random.default_rng(40630 + seed)
    ref, dist = _random_case(rng)[:2]
    f, h, w = ref.shape
    w8 = w - w % 8
    views = []
    for plane in (ref, dist):
        x0 = int(rng.integers(0, 64))
        pitch = x0 + w8 + int(rng.integers(0, 40))
        big = np.zeros((f, h, pitch), dtype=np.uint16)
        big[:, :, x0:x0 + w8] = plane[:, :, :w8]
        sl = (slice(None), slice(None), slice(x0, x0 + w8))
        views.append((big[sl], torch.from_numpy(big).cuda()[sl]))
    (rn, R), (dn, D) = views
    _in_place_case(rn, dn, R, D, 16)


def _random_case(rng):
    """A batch whose sums pass 2^53 (frames of 2^21 to 2^23 16-bit samples,
    mostly bright), with a random share and layout of dark samples: spread
    at random, in square blocks, or in whole rows; odd-only or any value."""
    share = float(rng.choice([0.0, 0.01, 0.05, 0.1, 0.3], p=[0.1, 0.2, 0.25, 0.25, 0.2]))
    lo = int(rng.choice([49152, 57344, 61440]))
    w = int(rng.integers(1400, 4097))
    need = int(1.05 * 2**53 / ((1 - share) * lo * lo)) + 1  # samples for the sums to pass 2^53
    h = int(rng.integers(-(-need // w), max(-(-need // w), 8_388_608 // w) + 1))
    nframes = int(rng.integers(1, 4))
    dark_max = int(rng.choice([255, 4095, 16383]))
    layout = rng.choice(["random", "blocks", "rows"])
    odd = bool(rng.integers(0, 2))
    planes = []
    for _ in range(2):
        bright = rng.integers(lo, 65535, size=(nframes, h, w), endpoint=True)
        dark = rng.integers(0, dark_max, size=(nframes, h, w), endpoint=True)
        if odd:
            dark |= 1
        if layout == "random":
            mask = rng.random((nframes, h, w)) < share
        elif layout == "blocks":
            b = 64
            cells = rng.random((nframes, -(-h // b), -(-w // b))) < share
            mask = np.repeat(np.repeat(cells, b, axis=1), b, axis=2)[:, :h, :w]
        else:
            mask = np.broadcast_to((rng.random((nframes, h, 1)) < share), (nframes, h, w))
        planes.append(np.where(mask, dark, bright).astype(np.uint16))
    return planes[0], planes[1], (w, h, nframes, lo, dark_max, share, str(layout), odd)


@pytest.mark.parametrize("seed", range(8))
def test_random_batches_past53(seed):
    """Seeded random sizes (unaligned frames too), frame counts and content
    mixes; bitwise against the sequential oracle on every frame and output."""
    rng = np.random.default_rng(20530 + seed)
    ref, dist, desc = _random_case(rng)
    past = check(ref, dist, 16)
    assert past > 0, f"case {desc} never passed 2^53"
