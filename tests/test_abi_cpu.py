"""The C ABI without a GPU: symbols, argument checks, host conclusions."""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle
from exact_reductions_amd import vqx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "vqx.h")


def _header_text():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(vqx_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return vqx.lib()


def test_library_exports_every_declared_symbol(L):
    declared = _declared_functions()
    assert declared == sorted(vqx.SYMBOLS)
    for name in declared:
        assert hasattr(L, name), name


def test_abi_version_matches_header(L):
    m = re.search(r"#define VQX_ABI_VERSION (\d+)", _header_text())
    assert vqx.abi_version() == int(m.group(1))


def test_status_codes_match_header():
    text = _header_text()
    for name, value in (("VQX_OK", 0), ("VQX_E_NULL", -1), ("VQX_E_DIMS", -2), ("VQX_E_BPC", -3),
                        ("VQX_E_NFRAMES", -4), ("VQX_E_ALIGN", -5), ("VQX_E_WORKSPACE", -6),
                        ("VQX_E_HIP", -7), ("VQX_E_NO_DEVICE", -8), ("VQX_E_STRIDE", -9),
                        ("VQX_E_PLANES", -10), ("VQX_E_SCRATCH", -11)):
        assert re.search(rf"\b{name} = {value}\b", text), name
    assert re.search(r"#define VQX_NOALLOC_SCRATCH_BYTES \(4u << 20\)", text)
    assert vqx.NOALLOC_SCRATCH_BYTES == 4 << 20
    for s in range(-11, 1):
        assert vqx.status_string(s) and vqx.status_string(s) != "unknown status"
    assert vqx.status_string(-99) == "unknown status"


def test_workspace_bytes():
    # one 64-byte record per workgroup
    # 3840x2160 uint16: 1 036 800 16-byte vectors, 2048 per workgroup -> 507 per frame
    assert vqx.plane_stats_workspace_bytes(3840, 2160, 16, 32) == 507 * 32 * 64
    # 576x324 uint8: 11 664 vectors -> 6 per frame
    assert vqx.plane_stats_workspace_bytes(576, 324, 8, 4) == 6 * 4 * 64
    assert vqx.plane_stats_workspace_bytes(1, 1, 12, 7) == 7 * 64
    for args, status in (((0, 5, 8, 1), vqx.E_DIMS), ((5, 0, 8, 1), vqx.E_DIMS),
                         ((8192, 4097, 8, 1), vqx.E_DIMS), ((5, 5, 7, 1), vqx.E_BPC),
                         ((5, 5, 17, 1), vqx.E_BPC), ((5, 5, 8, 0), vqx.E_NFRAMES)):
        with pytest.raises(vqx.VqxError) as e:
            vqx.plane_stats_workspace_bytes(*args)
        assert e.value.status == status
    assert vqx.lib().vqx_plane_stats_workspace_bytes(5, 5, 8, 1, None) == vqx.E_NULL


def test_largest_frame_accepted():
    assert vqx.plane_stats_workspace_bytes(8192, 4096, 16, 1) > 0   # exactly 2^25 pixels
    assert vqx.plane_stats_workspace_bytes(7680, 4320, 16, 1) > 0   # 8K


def test_batch_must_fit_one_dispatch():
    """A dispatch counts its work-items in 32 bits: at 256 per workgroup the
    widest launch, stage 1's, takes at most (2^32-1)//256 chunks, in the
    CPU-order form too.  1x1 frames are one chunk each."""
    top = (2**32 - 1) // 256
    assert vqx.plane_stats_workspace_bytes(1, 1, 16, top) == top * 64
    with pytest.raises(vqx.VqxError) as e:
        vqx.plane_stats_workspace_bytes(1, 1, 16, top + 1)
    assert e.value.status == vqx.E_NFRAMES
    assert vqx.plane_stats_cpu_order_workspace_bytes(1, 1, 16, top) > 0
    with pytest.raises(vqx.VqxError) as e:
        vqx.plane_stats_cpu_order_workspace_bytes(1, 1, 16, top + 1)
    assert e.value.status == vqx.E_NFRAMES
    # 4K 16-bit frames: 507 chunks each
    assert vqx.plane_stats_workspace_bytes(3840, 2160, 16, top // 507) > 0
    with pytest.raises(vqx.VqxError):
        vqx.plane_stats_workspace_bytes(3840, 2160, 16, top // 507 + 1)


class _Buffers:
    """Host memory standing in for device pointers: argument errors must be
    reported before any of it is touched."""

    def __init__(self):
        self.planes = np.zeros(4096, dtype=np.uint8)
        self.out = np.full(64, 0xFF, dtype=np.uint8)
        base = self.planes.ctypes.data
        self.ref = (base + 255) // 256 * 256
        self.dist = self.ref + 1024
        obase = self.out.ctypes.data
        self.noise = (obase + 7) // 8 * 8
        self.moments = self.noise + 8

    def untouched(self):
        return bool(np.all(self.out == 0xFF))


ARG_ERRORS = [
    ("null ref", dict(ref=0), vqx.E_NULL),
    ("null dist", dict(dist=0), vqx.E_NULL),
    ("null noise", dict(noise=0), vqx.E_NULL),
    ("null moments", dict(moments=0), vqx.E_NULL),
    ("w 0", dict(w=0), vqx.E_DIMS),
    ("h -1", dict(h=-1), vqx.E_DIMS),
    ("too many pixels", dict(w=8192, h=4097), vqx.E_DIMS),
    ("bpc 7", dict(bpc=7), vqx.E_BPC),
    ("bpc 17", dict(bpc=17), vqx.E_BPC),
    ("nframes 0", dict(nframes=0), vqx.E_NFRAMES),
    ("ref misaligned", dict(ref_off=8), vqx.E_ALIGN),
    ("dist misaligned", dict(dist_off=2), vqx.E_ALIGN),
    ("noise misaligned", dict(noise_off=4), vqx.E_ALIGN),
]


def _call(L, b, ws=None, ws_bytes=0, ref=None, dist=None, noise=None, moments=None, w=16, h=4,
          bpc=8, nframes=2, ref_off=0, dist_off=0, noise_off=0, noalloc=False):
    ref = b.ref + ref_off if ref is None else ref
    dist = b.dist + dist_off if dist is None else dist
    noise = b.noise + noise_off if noise is None else noise
    moments = b.moments if moments is None else moments
    if noalloc:
        return L.vqx_plane_stats_batch_noalloc(ref or None, dist or None, w, h, bpc, nframes,
                                               noise or None, moments or None, None)
    if ws is None:
        return L.vqx_plane_stats_batch(ref or None, dist or None, w, h, bpc, nframes,
                                       noise or None, moments or None, None)
    return L.vqx_plane_stats_batch_ws(ref or None, dist or None, w, h, bpc, nframes,
                                      noise or None, moments or None, ws or None, ws_bytes, None)


@pytest.mark.parametrize("name,kw,status", ARG_ERRORS, ids=[a[0] for a in ARG_ERRORS])
@pytest.mark.parametrize("form", ["self-allocating", "workspace", "no-alloc"])
def test_argument_errors_leave_outputs_untouched(L, name, kw, status, form):
    b = _Buffers()
    if form == "workspace":
        ws = np.zeros(4096, dtype=np.uint8)
        got = _call(L, b, ws=(ws.ctypes.data + 255) // 256 * 256, ws_bytes=1024, **kw)
    else:
        got = _call(L, b, noalloc=form == "no-alloc", **kw)
    assert got == status
    assert b.untouched()


def test_noalloc_scratch_limit(L):
    """A batch whose workspace exceeds the fixed scratch is rejected before
    any device call (so also without a device), outputs untouched; the
    largest batch that fits is not rejected for its size."""
    b = _Buffers()
    per_frame = vqx.plane_stats_workspace_bytes(3840, 2160, 16, 1)
    fits = vqx.NOALLOC_SCRATCH_BYTES // per_frame
    assert vqx.plane_stats_workspace_bytes(3840, 2160, 16, fits) <= vqx.NOALLOC_SCRATCH_BYTES
    assert _call(L, b, w=3840, h=2160, bpc=16, nframes=fits + 1, noalloc=True) == vqx.E_SCRATCH
    assert b.untouched()
    if not _has_gpu():
        assert _call(L, b, w=3840, h=2160, bpc=16, nframes=fits, noalloc=True) == vqx.E_NO_DEVICE
        assert b.untouched()


def test_cpu_order_arguments(L):
    b = _Buffers()
    ws = np.zeros(8192, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    need = vqx.plane_stats_cpu_order_workspace_bytes(16, 4, 8, 2)
    assert need >= vqx.plane_stats_workspace_bytes(16, 4, 8, 2)
    f = L.vqx_plane_stats_batch_cpu_order_ws
    assert f(b.ref, b.dist, 16, 4, 8, 2, b.noise, b.moments, None, b.moments, base, need, None) == vqx.E_NULL
    assert f(b.ref, b.dist, 16, 4, 8, 2, b.noise, b.moments, b.noise, b.moments + 4, base, need, None) == vqx.E_ALIGN
    assert f(b.ref, b.dist, 16, 4, 8, 2, b.noise, b.moments, b.noise, b.moments, base, need - 1, None) == vqx.E_WORKSPACE
    assert f(b.ref, b.dist, 0, 4, 8, 2, b.noise, b.moments, b.noise, b.moments, base, need, None) == vqx.E_DIMS
    assert b.untouched()
    with pytest.raises(vqx.VqxError):
        vqx.plane_stats_cpu_order_workspace_bytes(4, 4, 20, 1)


def test_read_probe_arguments(L):
    """The measurement probe checks its arguments like the timed entry point
    and queues nothing when they are wrong."""
    b = _Buffers()
    ws = np.zeros(4096, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    need = vqx.plane_stats_workspace_bytes(16, 4, 8, 2)
    f = L.vqx_read_probe_timed
    assert f(None, b.dist, 16, 4, 8, 2, base, need, None, None, None) == vqx.E_NULL
    assert f(b.ref, b.dist + 8, 16, 4, 8, 2, base, need, None, None, None) == vqx.E_ALIGN
    assert f(b.ref, b.dist, 16, 4, 8, 2, base, need - 1, None, None, None) == vqx.E_WORKSPACE
    assert f(b.ref, b.dist, 16, 4, 8, 2, None, need, None, None, None) == vqx.E_WORKSPACE
    assert f(b.ref, b.dist, 16, 0, 8, 2, base, need, None, None, None) == vqx.E_DIMS
    assert f(b.ref, b.dist, 16, 4, 17, 2, base, need, None, None, None) == vqx.E_BPC
    assert f(b.ref, b.dist, 16, 4, 8, 0, base, need, None, None, None) == vqx.E_NFRAMES
    assert np.all(ws == 0)


def test_workspace_errors(L):
    b = _Buffers()
    ws = np.zeros(4096, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    need = vqx.plane_stats_workspace_bytes(16, 4, 8, 2)
    assert _call(L, b, ws=base, ws_bytes=need - 1) == vqx.E_WORKSPACE
    assert _call(L, b, ws=base + 8, ws_bytes=need) == vqx.E_WORKSPACE
    assert L.vqx_plane_stats_batch_ws(b.ref, b.dist, 16, 4, 8, 2, b.noise, b.moments, None, need,
                                      None) == vqx.E_WORKSPACE
    assert b.untouched()


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="checks the no-device path")
def test_valid_call_without_device_reports_no_device(L):
    b = _Buffers()
    assert _call(L, b) == vqx.E_NO_DEVICE
    ws = np.zeros(4096, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    assert _call(L, b, ws=base, ws_bytes=1024) == vqx.E_NO_DEVICE
    assert _call(L, b, noalloc=True) == vqx.E_NO_DEVICE
    assert b.untouched()


# ------------------------------------------------------------------ conclusions

def _random_sums(rng, w, h, bpc, past53=False):
    pixels = w * h
    top = 255 if bpc == 8 else 65535
    q = oracle.q_int
    noise = int(rng.integers(0, pixels * q(top) + 1))
    r1 = int(rng.integers(0, pixels * top + 1))
    d1 = int(rng.integers(0, pixels * top + 1))
    r2 = int(rng.integers(0, pixels * q(top) + 1))
    d2 = int(rng.integers(0, pixels * q(top) + 1))
    if past53:
        r2 = int(rng.integers(1 << 53, pixels * q(top) + 1))
    return [noise, r1, d1, r2, d2]


@pytest.mark.parametrize("bpc", [8, 10, 12, 13, 16])
def test_conclusions_match_oracle_bitwise(bpc):
    rng = np.random.Generator(np.random.PCG64(bpc))
    for w, h in ((576, 324), (1920, 1080), (3840, 2160), (1, 1), (17, 3)):
        for _ in range(50):
            sums = _random_sums(rng, w, h, bpc, past53=(bpc == 16 and w * h > (1 << 21)))
            want = oracle.conclude_from_ints(sums, w, h, bpc)
            mse, db = vqx.conclude_psnr(sums[0], w, h, bpc, 0.0)
            assert mse == want[0]
            assert db == oracle.psnr_db(want[0], bpc, 0.0)
            got = vqx.conclude_moments(sums[1:], w, h, bpc)
            assert list(got) == list(want[1:])
            batch = vqx.conclude_batch([sums[0]], [sums[1:]], w, h, bpc, 60.0)
            assert list(batch[0]) == [want[0], oracle.psnr_db(want[0], bpc, 60.0)] + list(want[1:])


def test_psnr_textbook_values():
    # a constant 8-bit difference d gives mse = d^2 and PSNR = 20*log10(255/d)
    for d in (1, 2, 5, 255):
        mse, db = vqx.conclude_psnr(d * d * 100, 10, 10, 8)
        assert mse == d * d
        assert db == pytest.approx(20 * math.log10(255 / d), abs=1e-12)
    # peak on the 8-bit scale: (2^bpc - 1)/scaler
    _, db = vqx.conclude_psnr(16 * 16, 1, 1, 12)     # mse 1 on the 8-bit scale
    assert db == pytest.approx(20 * math.log10(4095 / 16), abs=1e-12)


def test_psnr_cap_and_zero_noise():
    assert vqx.conclude_psnr(0, 8, 8, 8, 60.0) == (0.0, 60.0)
    mse, db = vqx.conclude_psnr(0, 8, 8, 8, 0.0)
    assert mse == 0.0 and db == math.inf
    _, db = vqx.conclude_psnr(1, 1000, 1000, 8, 60.0)   # ~108 dB uncapped
    assert db == 60.0
    _, db = vqx.conclude_psnr(1, 1000, 1000, 8, 0.0)
    assert db > 100


def test_conclusion_errors():
    L = vqx.lib()
    out = np.zeros(24, dtype=np.float64)
    s = np.zeros(8, dtype=np.uint64)
    assert L.vqx_conclude_moments(None, 4, 4, 8, out.ctypes.data) == vqx.E_NULL
    assert L.vqx_conclude_moments(s.ctypes.data, 0, 4, 8, out.ctypes.data) == vqx.E_DIMS
    assert L.vqx_conclude_moments(s.ctypes.data, 4, 4, 18, out.ctypes.data) == vqx.E_BPC
    assert L.vqx_conclude_batch(s.ctypes.data, s.ctypes.data, 4, 4, 8, 0, 0.0, out.ctypes.data) == vqx.E_NFRAMES
    assert L.vqx_conclude_psnr(0, 4, 4, 7, 0.0, None, None) == vqx.E_BPC
    assert L.vqx_conclude_psnr(0, 4, 4, 8, 0.0, None, None) == vqx.OK
    assert np.all(out == 0)


def test_past53_conclusion_is_one_rounding():
    """Past 2^53 the conversion rounds once, to nearest even, like Python's
    int-to-float; the result stays within the page's bound of the exact mean."""
    w, h = 3840, 2160
    exact = (1 << 54) + 3          # odd, past 2^54: the conversion must round
    got = vqx.conclude_moments([0, 0, exact, 0], w, h, 16)[2]
    assert got == (float(exact) / 65536.0) / (w * h)
    from fractions import Fraction
    err = abs(Fraction(got) - Fraction(exact, 65536 * w * h))
    assert err <= oracle.past53_bound(w * h, 54, 16)


# ------------------------------------------------------------------ plane views

def test_view_workspace_bytes():
    # 3840x2160 16-bit: 4 rows per tile (4*3840 <= 2048*8), 540 tiles per frame
    assert vqx.plane_view_workspace_bytes(3840, 2160, 16, 32) == 540 * 32 * 64
    # rows longer than a tile are cut into segments of 2048 vectors
    assert vqx.plane_view_workspace_bytes(40000, 3, 16, 1) == 3 * 3 * 64
    assert vqx.plane_view_workspace_bytes(40000, 3, 8, 1) == 3 * 2 * 64
    assert vqx.plane_view_workspace_bytes(1, 1, 10, 5) == 5 * 64
    with pytest.raises(vqx.VqxError) as e:
        vqx.plane_view_workspace_bytes(1, 1, 10, (2**32 - 1) // 256 + 1)
    assert e.value.status == vqx.E_NFRAMES


VIEW_ERRORS = [
    ("null ref", dict(ref=0), vqx.E_NULL),
    ("null noise", dict(noise=0), vqx.E_NULL),
    ("w 0", dict(w=0), vqx.E_DIMS),
    ("bpc 17", dict(bpc=17), vqx.E_BPC),
    ("nframes 0", dict(nframes=0), vqx.E_NFRAMES),
    ("row stride below w", dict(rrs=15), vqx.E_STRIDE),
    ("negative frame stride", dict(dfs=-1), vqx.E_STRIDE),
    ("extent past 2^62 bytes", dict(rfs=2**62 - 8), vqx.E_STRIDE),
    ("16-bit extent past 2^62 bytes", dict(bpc=16, rfs=2**61), vqx.E_STRIDE),
    ("huge row stride", dict(drs=2**62), vqx.E_STRIDE),
    ("16-bit ref on an odd byte", dict(bpc=16, ref_off=1), vqx.E_ALIGN),
    ("noise misaligned", dict(noise_off=4), vqx.E_ALIGN),
]


def _view_call(L, b, fn, ws, ws_bytes, ref=None, noise=None, w=16, h=4, bpc=8, nframes=2, rrs=None, rfs=None,
               drs=None, dfs=None, ref_off=0, noise_off=0):
    ref = b.ref + ref_off if ref is None else ref
    noise = b.noise + noise_off if noise is None else noise
    rrs = w if rrs is None else rrs
    drs = w if drs is None else drs
    rfs = w * h if rfs is None else rfs
    dfs = w * h if dfs is None else dfs
    if fn == "stats":
        return L.vqx_plane_stats_view_ws(ref or None, rrs, rfs, b.dist, drs, dfs, w, h, bpc, nframes,
                                         noise or None, b.moments, ws, ws_bytes, None)
    return L.vqx_psnr_int_view_ws(ref or None, rrs, rfs, b.dist, drs, dfs, w, h, bpc, nframes,
                                  noise or None, ws, ws_bytes, None)


@pytest.mark.parametrize("name,kw,status", VIEW_ERRORS, ids=[a[0] for a in VIEW_ERRORS])
@pytest.mark.parametrize("fn", ["stats", "psnr_int"])
def test_view_argument_errors(L, name, kw, status, fn):
    b = _Buffers()
    ws = np.zeros(4096, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    assert _view_call(L, b, fn, base, 1024, **kw) == status
    assert b.untouched()


def test_view_workspace_and_moments_errors(L):
    b = _Buffers()
    ws = np.zeros(4096, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    need = vqx.plane_view_workspace_bytes(16, 4, 8, 2)
    for fn in ("stats", "psnr_int"):
        assert _view_call(L, b, fn, base, need - 1) == vqx.E_WORKSPACE
        assert _view_call(L, b, fn, base + 8, need) == vqx.E_WORKSPACE
        assert _view_call(L, b, fn, None, need) == vqx.E_WORKSPACE
    assert L.vqx_plane_stats_view_ws(b.ref, 16, 64, b.dist, 16, 64, 16, 4, 8, 2, b.noise, None, base, need,
                                     None) == vqx.E_NULL
    # an odd 8-bit base is fine; overlapping views (frame stride 0) are fine
    if not _has_gpu():
        assert _view_call(L, b, "stats", base, need, ref_off=1, rfs=0) == vqx.E_NO_DEVICE
    assert b.untouched()


@pytest.mark.parametrize("bpc", [8, 10, 12, 16])
def test_psnr_int_conclusion_matches_oracle_bitwise(bpc):
    rng = np.random.Generator(np.random.PCG64(100 + bpc))
    top = (1 << bpc) - 1
    for w, h in ((576, 324), (3840, 2160), (1, 1), (17, 3), (960, 540)):
        for _ in range(50):
            noise = int(rng.integers(0, w * h * top * top + 1))
            mse, db = vqx.conclude_psnr_int(noise, w, h, bpc, 0.0)
            assert mse == oracle.int_mse(noise, w, h)
            assert db == oracle.int_psnr_db(noise, w, h, bpc, 0.0)
            _, capped = vqx.conclude_psnr_int(noise, w, h, bpc, 6.0 * bpc + 12.0)
            assert capped == oracle.int_psnr_db(noise, w, h, bpc, 6.0 * bpc + 12.0)
    assert vqx.conclude_psnr_int(0, 4, 4, bpc, 0.0)[1] == math.inf
    assert vqx.conclude_psnr_int(0, 4, 4, bpc, 50.0) == (0.0, 50.0)
    # past 2^53: one rounding of the integer, then the division
    big = (1 << 55) + 1
    assert vqx.conclude_psnr_int(big, 7680, 4320, 16)[0] == float(big) / (7680 * 4320)
    noises = [int(v) for v in rng.integers(0, 1920 * 1080 * top * top + 1, size=7)] + [0]
    batch = vqx.conclude_psnr_int_batch(noises, 1920, 1080, bpc, 50.0)
    for k, n in enumerate(noises):
        assert list(batch[k]) == [oracle.int_mse(n, 1920, 1080), oracle.int_psnr_db(n, 1920, 1080, bpc, 50.0)]
    out = np.zeros(4)
    L = vqx.lib()
    assert L.vqx_conclude_psnr_int_batch(None, 4, 4, 8, 1, 0.0, out.ctypes.data) == vqx.E_NULL
    assert L.vqx_conclude_psnr_int_batch(np.zeros(2, np.uint64).ctypes.data, 4, 4, 8, 0, 0.0,
                                         out.ctypes.data) == vqx.E_NFRAMES
    assert vqx.lib().vqx_conclude_psnr_int(0, 0, 4, 8, 0.0, None, None) == vqx.E_DIMS
    assert vqx.lib().vqx_conclude_psnr_int(0, 4, 4, 17, 0.0, None, None) == vqx.E_BPC


# ------------------------------------------------------------ host-fed batches

def test_host_workspace_bytes():
    up = lambda x: (x + 255) // 256 * 256
    # two staging slots of 4 frames of both planes, then 4 frames of records
    plane = 3840 * 2160 * 2 * 4
    assert vqx.plane_stats_host_workspace_bytes(3840, 2160, 16, 4) == up(4 * up(plane) + 507 * 4 * 64)
    # 17x9 8-bit: 153 bytes per frame and plane, one chunk per frame
    assert vqx.plane_stats_host_workspace_bytes(17, 9, 8, 3) == up(4 * up(153 * 3) + 3 * 64)
    with pytest.raises(vqx.VqxError) as e:
        vqx.plane_stats_host_workspace_bytes(17, 9, 8, 0)
    assert e.value.status == vqx.E_NFRAMES


def test_host_argument_errors(L):
    b = _Buffers()
    ws = np.zeros(8192, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    need = vqx.plane_stats_host_workspace_bytes(16, 4, 8, 2)
    f = L.vqx_plane_stats_host_ws
    host = np.zeros(16 * 4 * 5, dtype=np.uint8)
    h = host.ctypes.data
    cases = [
        ((None, h, 16, 4, 8, 5, 2, b.noise, b.moments, base, need, None, None), vqx.E_NULL),
        ((h, h, 16, 4, 8, 5, 2, b.noise, None, base, need, None, None), vqx.E_NULL),
        ((h, h, 0, 4, 8, 5, 2, b.noise, b.moments, base, need, None, None), vqx.E_DIMS),
        ((h, h, 16, 4, 7, 5, 2, b.noise, b.moments, base, need, None, None), vqx.E_BPC),
        ((h, h, 16, 4, 8, 0, 2, b.noise, b.moments, base, need, None, None), vqx.E_NFRAMES),
        ((h, h, 16, 4, 8, 5, 0, b.noise, b.moments, base, need, None, None), vqx.E_NFRAMES),
        ((h, h, 16, 4, 8, 5, 2, b.noise + 4, b.moments, base, need, None, None), vqx.E_ALIGN),
        ((h, h, 16, 4, 8, 5, 2, b.noise, b.moments, base, need - 1, None, None), vqx.E_WORKSPACE),
        ((h, h, 16, 4, 8, 5, 2, b.noise, b.moments, base + 8, need, None, None), vqx.E_WORKSPACE),
        ((h, h, 16, 4, 8, 5, 2, b.noise, b.moments, None, need, None, None), vqx.E_WORKSPACE),
    ]
    for args, status in cases:
        assert f(*args) == status, (args, status)
    assert b.untouched()
    if not _has_gpu():
        assert f(h, h, 16, 4, 8, 5, 2, b.noise, b.moments, base, need, None, None) == vqx.E_NO_DEVICE
        assert b.untouched()


def _pairs(b, sizes, rrs=None, off=0):
    arr = (vqx.PlanePair * len(sizes))()
    for k, (w, h) in enumerate(sizes):
        arr[k] = vqx.PlanePair(b.ref + off, rrs or w, w * h, b.dist, w, w * h, w, h)
    return arr


def test_planes_workspace_and_errors(L):
    """Several planes: the workspace is the sum of the planes' view
    workspaces; argument errors are reported before anything is queued."""
    sizes = [(1920, 1080), (960, 540), (960, 540)]
    want = sum(vqx.plane_view_workspace_bytes(w, h, 10, 7) for w, h in sizes)
    assert vqx.planes_workspace_bytes(sizes, 10, 7) == want
    with pytest.raises(vqx.VqxError) as e:
        vqx.planes_workspace_bytes([(4, 4)] * 5, 10, 1)
    assert e.value.status == vqx.E_PLANES
    with pytest.raises(vqx.VqxError) as e:
        vqx.planes_workspace_bytes([], 10, 1)
    assert e.value.status == vqx.E_PLANES
    with pytest.raises(vqx.VqxError) as e:
        vqx.planes_workspace_bytes([(4, 4), (0, 4)], 10, 1)
    assert e.value.status == vqx.E_DIMS
    # all planes' tiles share one dispatch: (2^32-1)/256 in all
    top = (2**32 - 1) // 256
    assert vqx.planes_workspace_bytes([(1, 1)], 16, top) > 0
    with pytest.raises(vqx.VqxError) as e:
        vqx.planes_workspace_bytes([(1, 1), (1, 1)], 16, top // 2 + 1)
    assert e.value.status == vqx.E_NFRAMES

    b = _Buffers()
    ws = np.zeros(8192, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    small = [(16, 4), (8, 2)]
    need = vqx.planes_workspace_bytes(small, 10, 2)
    f = L.vqx_psnr_int_planes_ws
    g = L.vqx_plane_stats_planes_ws
    ok = _pairs(b, small)
    assert f(None, 2, 10, 2, b.noise, base, need, None) == vqx.E_NULL
    assert f(ok, 2, 10, 2, None, base, need, None) == vqx.E_NULL
    assert g(ok, 2, 10, 2, b.noise, None, base, need, None) == vqx.E_NULL
    assert f(ok, 0, 10, 2, b.noise, base, need, None) == vqx.E_PLANES
    assert f(ok, 5, 10, 2, b.noise, base, need, None) == vqx.E_PLANES
    assert f(ok, 2, 7, 2, b.noise, base, need, None) == vqx.E_BPC
    assert f(ok, 2, 10, 0, b.noise, base, need, None) == vqx.E_NFRAMES
    assert f(_pairs(b, small, rrs=3), 2, 10, 2, b.noise, base, need, None) == vqx.E_STRIDE
    assert f(_pairs(b, small, off=1), 2, 10, 2, b.noise, base, need, None) == vqx.E_ALIGN
    assert f(ok, 2, 10, 2, b.noise + 4, base, need, None) == vqx.E_ALIGN
    assert f(ok, 2, 10, 2, b.noise, base, need - 1, None) == vqx.E_WORKSPACE
    assert g(ok, 2, 10, 2, b.noise, b.moments, base + 8, need, None) == vqx.E_WORKSPACE
    nul = _pairs(b, small)
    nul[1].dist = None
    assert f(nul, 2, 10, 2, b.noise, base, need, None) == vqx.E_NULL
    assert b.untouched() and np.all(ws == 0)


def test_view_cpu_order_workspace_and_errors(L):
    """The CPU-order form over views: its workspace holds the contiguous
    form's and both planes of the batch; argument errors are reported before
    anything is queued."""
    need = vqx.plane_stats_view_cpu_order_workspace_bytes(3840, 2160, 16, 2)
    assert need >= vqx.plane_stats_cpu_order_workspace_bytes(3840, 2160, 16, 2) + 2 * 3840 * 2160 * 2 * 2
    b = _Buffers()
    ws = np.zeros(16384, dtype=np.uint8)
    base = (ws.ctypes.data + 255) // 256 * 256
    need = vqx.plane_stats_view_cpu_order_workspace_bytes(16, 4, 10, 2)
    f = L.vqx_plane_stats_view_cpu_order_ws
    args = lambda **kw: [kw.get("ref", b.ref), kw.get("rrs", 16), kw.get("rfs", 64), kw.get("dist", b.dist),
                         kw.get("drs", 16), kw.get("dfs", 64), 16, 4, kw.get("bpc", 10), 2, kw.get("noise", b.noise),
                         b.moments, kw.get("cn", b.noise), b.moments, base, kw.get("ws", need), None]
    assert f(*args(ref=None)) == vqx.E_NULL
    assert f(*args(cn=None)) == vqx.E_NULL
    assert f(*args(bpc=17)) == vqx.E_BPC
    assert f(*args(rrs=15)) == vqx.E_STRIDE
    assert f(*args(dfs=-1)) == vqx.E_STRIDE
    assert f(*args(dist=b.dist + 1)) == vqx.E_ALIGN
    assert f(*args(cn=b.noise + 4)) == vqx.E_ALIGN
    assert f(*args(ws=need - 1)) == vqx.E_WORKSPACE
    assert b.untouched() and np.all(ws == 0)
