"""Plane views and the integer psnr twin on the device (marked gpu).

Every case builds its planes as views of larger tensors (a padded pitch, a
region of interest, one plane of planar YUV frames), runs
``vqx_plane_stats_view_ws`` and ``vqx_psnr_int_view_ws`` through the C ABI,
and compares element by element with the oracle applied to the same samples
(numpy slices): the five exact sums with O2, the integer noise with O3, the
integer psnr conclusion with O3's.
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


def _dtype(bpc):
    return np.uint8 if bpc == 8 else np.uint16


def _rand(rng, shape, bpc, lo=0, hi=None):
    hi = (1 << bpc) - 1 if hi is None else hi
    return rng.integers(lo, hi, size=shape, endpoint=True).astype(_dtype(bpc))


def check_views(ref_np, dist_np, ref_dev, dist_dev, bpc, label=""):
    """ref_np/dist_np: [F][h][w] numpy views of the samples that the device
    views ref_dev/dist_dev select."""
    f = ref_np.shape[0]
    h, w = ref_np.shape[1:]
    noise, moments = vqx.plane_stats_view(ref_dev, dist_dev, bpc)
    inoise = vqx.psnr_int_view(ref_dev, dist_dev, bpc)
    torch.cuda.synchronize()
    noise, moments, inoise = noise.cpu().numpy(), moments.cpu().numpy(), inoise.cpu().numpy()
    for k in range(f):
        r = np.ascontiguousarray(ref_np[k])
        d = np.ascontiguousarray(dist_np[k])
        want = oracle.exact_frame_sums(r, d)
        got = [int(noise[k])] + [int(v) for v in moments[k]]
        assert got == list(want), f"{label} frame {k}: five sums"
        wn = oracle.int_noise(r, d)
        assert int(inoise[k]) == wn, f"{label} frame {k}: integer noise"
        assert vqx.conclude_psnr_int(int(inoise[k]), w, h, bpc, 0.0)[1] == oracle.int_psnr_db(wn, w, h, bpc)
    return noise, moments, inoise


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_contiguous_workloads_as_views(n):
    """A contiguous batch is the view with row stride w and frame stride w*h;
    the results equal those of the contiguous entry point too."""
    wl = synth.WORKLOADS[n]
    ref, dist = synth.generate(n, nframes=min(wl.nframes, 6))
    r = torch.from_numpy(ref).cuda()
    d = torch.from_numpy(dist).cuda()
    noise, moments, _ = check_views(ref, dist, r, d, wl.bpc, f"workload {n}")
    n2, m2 = vqx.plane_stats_batch(r, d, wl.bpc)
    torch.cuda.synchronize()
    assert (n2.cpu().numpy() == noise).all() and (m2.cpu().numpy() == moments).all()


@pytest.mark.parametrize("bpc", [8, 10, 16])
@pytest.mark.parametrize("w,h,pitch,x0,y0", [
    (1920, 1080, 2048, 0, 0),      # padded pitch, rows 16-byte aligned
    (1920, 1080, 1920 + 64, 32, 8),  # a region of interest, aligned
    (1000, 301, 1037, 3, 5),       # odd pitch: rows at varying offsets
    (333, 77, 400, 7, 1),          # region starting mid-vector
    (7, 9, 13, 1, 2),              # narrower than a vector
    (1, 1, 1, 0, 0),
])
def test_pitched_regions(bpc, w, h, pitch, x0, y0):
    rng = np.random.default_rng(w * 31 + pitch + bpc)
    f = 3
    big_r = _rand(rng, (f, h + y0 + 2, pitch + x0), bpc, hi=255 if bpc == 8 else 65535)
    big_d = _rand(rng, (f, h + y0 + 2, pitch + x0), bpc, hi=255 if bpc == 8 else 65535)
    sl = (slice(None), slice(y0, y0 + h), slice(x0, x0 + w))
    R = torch.from_numpy(big_r).cuda()
    D = torch.from_numpy(big_d).cuda()
    check_views(big_r[sl], big_d[sl], R[sl], D[sl], bpc, f"{w}x{h} pitch {pitch} at ({x0},{y0})")


@pytest.mark.parametrize("bpc", [8, 10])
@pytest.mark.parametrize("chroma", ["420", "422", "444"])
def test_planar_yuv_frames(bpc, chroma):
    """Y, U and V of each frame stored one after another, frames one after
    another: each plane is a view with its own row stride, a frame stride of
    the whole frame, and a base offset."""
    w, h, f = 1920, 1080, 4
    cw = w // 2 if chroma in ("420", "422") else w
    ch = h // 2 if chroma == "420" else h
    sizes = [w * h, cw * ch, cw * ch]
    frame = sum(sizes)
    rng = np.random.default_rng(hash(chroma) % 1000 + bpc)
    buf_r = _rand(rng, (f, frame), bpc)
    buf_d = buf_r.astype(np.int64) + rng.integers(-20, 20, size=buf_r.shape, endpoint=True)
    buf_d = np.clip(buf_d, 0, (1 << bpc) - 1).astype(_dtype(bpc))
    R = torch.from_numpy(buf_r).cuda()
    D = torch.from_numpy(buf_d).cuda()
    off = 0
    for p, (pw, ph) in enumerate(((w, h), (cw, ch), (cw, ch))):
        rv = torch.as_strided(R, (f, ph, pw), (frame, pw, 1), off)
        dv = torch.as_strided(D, (f, ph, pw), (frame, pw, 1), off)
        rn = np.lib.stride_tricks.as_strided(buf_r.reshape(-1)[off:], (f, ph, pw),
                                             (frame * buf_r.itemsize, pw * buf_r.itemsize, buf_r.itemsize))
        dn = np.lib.stride_tricks.as_strided(buf_d.reshape(-1)[off:], (f, ph, pw),
                                             (frame * buf_d.itemsize, pw * buf_d.itemsize, buf_d.itemsize))
        check_views(rn, dn, rv, dv, bpc, f"{chroma} plane {p}")
        off += sizes[p]


def test_ref_and_dist_at_different_offsets():
    """ref contiguous, dist in a pitched buffer one sample off: their vectors
    do not pair, and the tile is read sample by sample."""
    rng = np.random.default_rng(41)
    f, h, w = 2, 300, 1000
    ref = _rand(rng, (f, h, w), 16, hi=65535)
    big = _rand(rng, (f, h, w + 9), 16, hi=65535)
    dist = big[:, :, 1:1 + w]
    check_views(ref, dist, torch.from_numpy(ref).cuda(), torch.from_numpy(big).cuda()[:, :, 1:1 + w], 16)


@pytest.mark.parametrize("bpc", [8, 10, 16])
@pytest.mark.parametrize("pitch,xr,xd", [(2048, 0, 1), (2048, 3, 0), (2051, 1, 6), (2049, 0, 5), (2048, 7, 2)])
def test_ref_and_dist_offsets_apart_one_pitch(bpc, pitch, xr, xd):
    """ref and dist in buffers of one pitch at different column offsets: in
    every row dist starts the same distance past ref within 16 bytes, and
    its vectors are cut from aligned blocks (even and odd pitches, dist
    before or after ref, at every depth)."""
    rng = np.random.default_rng(pitch * 7 + xr * 3 + xd + bpc)
    f, h, w = 2, 70, 1900
    big_r = _rand(rng, (f, h + 2, pitch), bpc)
    big_d = _rand(rng, (f, h + 2, pitch), bpc)
    sr = (slice(None), slice(1, 1 + h), slice(xr, xr + w))
    sd = (slice(None), slice(2, 2 + h), slice(xd, xd + w))
    check_views(big_r[sr], big_d[sd], torch.from_numpy(big_r).cuda()[sr], torch.from_numpy(big_d).cuda()[sd], bpc,
                f"pitch {pitch} ref at {xr}, dist at {xd}")


@pytest.mark.parametrize("bpc,w", [(16, 256), (8, 512)])
@pytest.mark.parametrize("ref_max", [True, False])
def test_row_path_budget_at_max_values(bpc, w, ref_max):
    """Rows of 32 vectors (the narrowest the row-by-row path takes) give 64
    rows per tile, so a lane adds up to 64 whole vectors and 64 edge samples.
    Every sample of one plane is the largest value and the other plane is
    zero: each square sum of the tile is at its budget.  ref and dist start
    at different offsets within 16 bytes (and at 8 bits the pitch, 522
    bytes, moves every row to another offset), so every tile is read row by
    row; 197 rows make three whole tiles and a ragged one."""
    f, h = 2, 197
    pitch = w + 7 + (1 if bpc == 16 else 3)
    top = (1 << bpc) - 1
    big_r = np.full((f, h, pitch), top if ref_max else 0, dtype=_dtype(bpc))
    big_d = np.full((f, h, pitch), 0 if ref_max else top, dtype=_dtype(bpc))
    sr = (slice(None), slice(None), slice(1, 1 + w))
    sd = (slice(None), slice(None), slice(6, 6 + w))
    check_views(big_r[sr], big_d[sd], torch.from_numpy(big_r).cuda()[sr], torch.from_numpy(big_d).cuda()[sd], bpc,
                f"w {w} bpc {bpc}")


@pytest.mark.parametrize("bpc,w", [(16, 40000), (8, 70000), (16, 16384), (16, 16385)])
def test_rows_longer_than_a_tile(bpc, w):
    rng = np.random.default_rng(w)
    f, h = 2, 3
    big_r = _rand(rng, (f, h, w + 5), bpc)
    big_d = _rand(rng, (f, h, w + 5), bpc)
    sl = (slice(None), slice(None), slice(2, 2 + w))
    check_views(big_r[sl], big_d[sl], torch.from_numpy(big_r).cuda()[sl],
                torch.from_numpy(big_d).cuda()[sl], bpc, f"w {w}")


def test_frame_stride_zero():
    """Every frame reads the same plane."""
    rng = np.random.default_rng(3)
    ref = _rand(rng, (1, 64, 80), 12)
    dist = _rand(rng, (1, 64, 80), 12)
    R = torch.from_numpy(ref).cuda().expand(5, 64, 80)
    D = torch.from_numpy(dist).cuda().expand(5, 64, 80)
    assert R.stride(0) == 0
    noise, moments, inoise = check_views(np.broadcast_to(ref, (5, 64, 80)), np.broadcast_to(dist, (5, 64, 80)),
                                         R, D, 12, "stride 0")
    assert len(set(int(v) for v in inoise)) == 1


def test_integer_noise_differs_from_float_past_4096():
    """16-bit differences above 4096: the float square rounds, the integer
    one does not -- e.g. 4097^2 = 2^24 + 8193 vs its float square 16 785 408."""
    f, h, w = 2, 1080, 1920
    ref = np.full((f, h, w), 4097 + 500, dtype=np.uint16)
    dist = np.full((f, h, w), 500, dtype=np.uint16)
    R, D = torch.from_numpy(ref).cuda(), torch.from_numpy(dist).cuda()
    noise, _, inoise = check_views(ref, dist, R, D, 16)
    assert int(inoise[0]) - int(noise[0]) == w * h
    rng = np.random.default_rng(9)
    ref = _rand(rng, (f, h, w), 16, hi=65535)
    dist = _rand(rng, (f, h, w), 16, hi=65535)
    noise, _, inoise = check_views(ref, dist, torch.from_numpy(ref).cuda(), torch.from_numpy(dist).cuda(), 16)
    assert (inoise != noise).all()


def test_largest_frame_pitched():
    rng = np.random.default_rng(8192)
    big_r = _rand(rng, (1, 4096, 8192 + 64), 16, hi=65535)
    big_d = _rand(rng, (1, 4096, 8192 + 64), 16, hi=65535)
    sl = (slice(None), slice(None), slice(64, 64 + 8192))
    check_views(big_r[sl], big_d[sl], torch.from_numpy(big_r).cuda()[sl], torch.from_numpy(big_d).cuda()[sl], 16)


def test_outputs_written_not_accumulated():
    rng = np.random.default_rng(12)
    ref = _rand(rng, (3, 50, 70), 10)
    dist = _rand(rng, (3, 50, 70), 10)
    R, D = torch.from_numpy(ref).cuda(), torch.from_numpy(dist).cuda()
    f, h, w = ref.shape
    L = vqx.lib()
    out = torch.full((6 * f,), -1, dtype=torch.int64, device="cuda")
    ws = torch.full((vqx.plane_view_workspace_bytes(w, h, 10, f),), 0xFF, dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert L.vqx_plane_stats_view_ws(R.data_ptr(), w, w * h, D.data_ptr(), w, w * h, w, h, 10, f,
                                         out[:f].data_ptr(), out[f:5 * f].data_ptr(), ws.data_ptr(),
                                         ws.numel(), st) == 0
        assert L.vqx_psnr_int_view_ws(R.data_ptr(), w, w * h, D.data_ptr(), w, w * h, w, h, 10, f,
                                      out[5 * f:].data_ptr(), ws.data_ptr(), ws.numel(), st) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for k in range(f):
        want = oracle.exact_frame_sums(ref[k], dist[k])
        assert [int(o[k])] + [int(v) for v in o[f + 4 * k:f + 4 * k + 4]] == list(want)
        assert int(o[5 * f + k]) == oracle.int_noise(ref[k], dist[k])


@pytest.mark.parametrize("seed", range(10))
def test_random_views(seed):
    """Seeded random views: depth, size, pitch, offsets, frame count and
    frame stride (0 or the buffer's), half of them rows of whole aligned
    vectors (read with the contiguous chunks at two-byte samples), half at
    any offset (read in row tiles); against the oracle and the contiguous
    entry point on the copied samples."""
    rng = np.random.default_rng(7100 + seed)
    aligned = seed % 2 == 0
    bpc = int(rng.integers(9, 17)) if aligned else int(rng.integers(8, 17))
    if aligned:
        w = 8 * int(rng.integers(1, 500))
        pitch = w + 8 * int(rng.integers(0, 12))
        x0 = 8 * int(rng.integers(0, 4))
    else:
        w = int(rng.integers(1, 3000))
        pitch = w + int(rng.integers(0, 40))
        x0 = int(rng.integers(0, 20))
    h = int(rng.integers(1, 300))
    y0 = int(rng.integers(0, 4))
    f = int(rng.integers(1, 5))
    same_plane = bool(rng.integers(0, 4) == 0)
    hi = (1 << bpc) - 1
    fb = 1 if same_plane else f
    big_r = _rand(rng, (fb, h + y0 + 1, pitch + x0), bpc, lo=hi // 3)
    noise = rng.integers(-300, 300, size=big_r.shape, endpoint=True)
    big_d = np.clip(big_r.astype(np.int64) + noise, 0, hi).astype(_dtype(bpc))
    sl = (slice(None), slice(y0, y0 + h), slice(x0, x0 + w))
    R, D = torch.from_numpy(big_r).cuda()[sl], torch.from_numpy(big_d).cuda()[sl]
    rn, dn = big_r[sl], big_d[sl]
    if same_plane:
        R, D = R.expand(f, h, w), D.expand(f, h, w)
        rn, dn = np.broadcast_to(rn, (f, h, w)), np.broadcast_to(dn, (f, h, w))
    label = f"seed {seed}: bpc {bpc} {w}x{h}x{f} pitch {pitch} at ({x0},{y0}) same_plane {same_plane}"
    noise_v, moments_v, _ = check_views(rn, dn, R, D, bpc, label)
    n2, m2 = vqx.plane_stats_batch(torch.from_numpy(np.ascontiguousarray(rn)).cuda(),
                                   torch.from_numpy(np.ascontiguousarray(dn)).cuda(), bpc)
    torch.cuda.synchronize()
    assert (n2.cpu().numpy() == noise_v).all() and (m2.cpu().numpy() == moments_v).all(), label


# ------------------------------------------------------------ several planes
def check_planes(pairs_np, pairs_dev, bpc, label=""):
    """pairs_np: [(ref [F][h][w], dist)] numpy views of what pairs_dev select.
    Both several-planes entry points against the oracle, plane by plane,
    and against the one-plane entry points."""
    noise, moments = vqx.plane_stats_planes(pairs_dev, bpc)
    inoise = vqx.psnr_int_planes(pairs_dev, bpc)
    torch.cuda.synchronize()
    noise, moments, inoise = noise.cpu().numpy(), moments.cpu().numpy(), inoise.cpu().numpy()
    for p, ((rn, dn), (rd, dd)) in enumerate(zip(pairs_np, pairs_dev)):
        f = rn.shape[0]
        for k in range(f):
            r = np.ascontiguousarray(rn[k])
            d = np.ascontiguousarray(dn[k])
            want = oracle.exact_frame_sums(r, d)
            got = [int(noise[p, k])] + [int(v) for v in moments[p, k]]
            assert got == list(want), f"{label} plane {p} frame {k}: five sums"
            assert int(inoise[p, k]) == oracle.int_noise(r, d), f"{label} plane {p} frame {k}: integer noise"
        n1, m1 = vqx.plane_stats_view(rd, dd, bpc)
        i1 = vqx.psnr_int_view(rd, dd, bpc)
        torch.cuda.synchronize()
        assert (n1.cpu().numpy() == noise[p]).all() and (m1.cpu().numpy() == moments[p]).all()
        assert (i1.cpu().numpy() == inoise[p]).all()
    return noise, moments, inoise


@pytest.mark.parametrize("bpc", [8, 10, 16])
@pytest.mark.parametrize("chroma", ["420", "422", "444"])
def test_planes_of_planar_yuv(bpc, chroma):
    """Y, U and V of planar frames in one call of each entry point."""
    w, h, f = 1920, 1080, 3
    sx, sy = synth.CHROMA[chroma]
    cw, ch = -(-w // sx), -(-h // sy)
    sizes = [w * h, cw * ch, cw * ch]
    frame = sum(sizes)
    rng = np.random.default_rng(bpc * 7 + sx * 3 + sy)
    buf_r = _rand(rng, (f, frame), bpc)
    buf_d = np.clip(buf_r.astype(np.int64) + rng.integers(-300, 300, size=buf_r.shape, endpoint=True), 0,
                    (1 << bpc) - 1).astype(_dtype(bpc))
    R = torch.from_numpy(buf_r).cuda()
    D = torch.from_numpy(buf_d).cuda()
    off, pairs_np, pairs_dev = 0, [], []
    for pw, ph, size in ((w, h, sizes[0]), (cw, ch, sizes[1]), (cw, ch, sizes[2])):
        pairs_dev.append((torch.as_strided(R, (f, ph, pw), (frame, pw, 1), off),
                          torch.as_strided(D, (f, ph, pw), (frame, pw, 1), off)))
        pairs_np.append(tuple(np.lib.stride_tricks.as_strided(
            b.reshape(-1)[off:], (f, ph, pw), (frame * b.itemsize, pw * b.itemsize, b.itemsize))
            for b in (buf_r, buf_d)))
        off += size
    check_planes(pairs_np, pairs_dev, bpc, f"{chroma} {bpc}-bit")


def test_planes_of_mixed_shapes():
    """Four planes of unlike shapes and layouts: a pitched region, a row
    longer than a tile, a 1x1 plane, and a plane whose ref and dist sit at
    different offsets within 16 bytes."""
    rng = np.random.default_rng(77)
    f = 2
    big_r = _rand(rng, (f, 300, 1100), 16)
    big_d = _rand(rng, (f, 300, 1100), 16)
    long_r = _rand(rng, (f, 2, 20000), 16)
    long_d = _rand(rng, (f, 2, 20000), 16)
    one_r = _rand(rng, (f, 1, 1), 16)
    one_d = _rand(rng, (f, 1, 1), 16)
    odd_r = _rand(rng, (f, 40, 70), 16)
    odd_d = _rand(rng, (f, 40, 73), 16)
    regions = [
        ((big_r, big_d), (slice(None), slice(5, 290), slice(3, 1003))),
        ((long_r, long_d), (slice(None), slice(None), slice(1, 19999))),
        ((one_r, one_d), (slice(None), slice(None), slice(None))),
    ]
    pairs_np, pairs_dev = [], []
    for (r, d), sl in regions:
        pairs_np.append((r[sl], d[sl]))
        pairs_dev.append((torch.from_numpy(r).cuda()[sl], torch.from_numpy(d).cuda()[sl]))
    pairs_np.append((odd_r, odd_d[:, :, 3:]))
    pairs_dev.append((torch.from_numpy(odd_r).cuda(), torch.from_numpy(odd_d).cuda()[:, :, 3:]))
    check_planes(pairs_np, pairs_dev, 16, "mixed")


def test_one_plane_and_outputs_written():
    """One plane through the several-planes form equals the view form, and
    the outputs are written, not added to (pre-filled outputs and workspace,
    two calls in a row)."""
    rng = np.random.default_rng(5)
    ref = _rand(rng, (3, 50, 70), 12)
    dist = _rand(rng, (3, 50, 70), 12)
    R, D = torch.from_numpy(ref).cuda(), torch.from_numpy(dist).cuda()
    check_planes([(ref, dist)], [(R, D)], 12, "one plane")
    arr, keep, f = vqx.plane_pairs([(R, D), (R[:, ::2, :], D[:, ::2, :])], 12)
    need = vqx.planes_workspace_bytes([(70, 50), (70, 25)], 12, 3)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((2 * 3 + 2 * 3 * 5,), -1, dtype=torch.int64, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    L = vqx.lib()
    for _ in range(2):
        assert L.vqx_psnr_int_planes_ws(arr, 2, 12, 3, out[:6].data_ptr(), ws.data_ptr(), need, st) == 0
        assert L.vqx_plane_stats_planes_ws(arr, 2, 12, 3, out[6:12].data_ptr(), out[12:].data_ptr(), ws.data_ptr(),
                                           need, st) == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    for p, (r, d) in enumerate(((ref, dist), (ref[:, ::2, :], dist[:, ::2, :]))):
        for k in range(3):
            rk, dk = np.ascontiguousarray(r[k]), np.ascontiguousarray(d[k])
            assert int(o[3 * p + k]) == oracle.int_noise(rk, dk)
            want = oracle.exact_frame_sums(rk, dk)
            assert int(o[6 + 3 * p + k]) == want[0]
            assert [int(v) for v in o[12 + 4 * (3 * p + k):12 + 4 * (3 * p + k) + 4]] == list(want[1:])
