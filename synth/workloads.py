"""Seeded synthetic luma-plane workloads.

This module only draws random sample values.  It computes none of the
reductions: the oracle and the HIP library both receive the arrays it returns
and nothing else from here.

Layout of every batch: a C-contiguous numpy array ``[nframes][h][w]`` of
``uint8`` (8 bits per component) or ``uint16`` (9..16 bits, value in the low
bits), one array for the reference planes and one for the distorted planes.

The first five named workloads stand in for the clips the pages measure on
(Netflix 576x324, BBB and the checkerboards at 1920x1080 and 3840x2160,
full-range noise and the bright 16-bit pair), none of which exists here; the
sixth for the 2560x1440 frame whose sums pass 2**53 units, with dark samples
whose squares are not multiples of the binade's unit.  Each workload
has one ``numpy.random.Generator(PCG64(1000 + number))``; frames are drawn in
order, for each frame first the reference plane, then the distorted plane.
"Uniform a..b" below means integers with both ends included; "rint" is
``numpy.rint`` (ties to even).
"""

from __future__ import annotations

import dataclasses
import hashlib

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    number: int
    name: str
    w: int
    h: int
    nframes: int
    bpc: int
    recipe: str

    @property
    def dtype(self):
        return np.uint8 if self.bpc == 8 else np.uint16

    @property
    def bytes_per_sample(self) -> int:
        return 1 if self.bpc == 8 else 2

    @property
    def bytes_per_frame(self) -> int:
        """Bytes read per frame: both planes, each read once."""
        return 2 * self.w * self.h * self.bytes_per_sample

    @property
    def seed(self) -> int:
        return 1000 + self.number


WORKLOADS = {
    1: Workload(1, "576x324 8-bit", 576, 324, 4, 8,
                "ref uniform 0..255; dist = clip(ref + rint(N(0,8)), 0, 255)"),
    2: Workload(2, "1920x1080 10-bit", 1920, 1080, 48, 10,
                "ref = clip(rint(1023*(x/(w-1) + y/(h-1))/2 + N(0,40)), 0, 1023) "
                "(a diagonal ramp with texture redrawn per frame); "
                "dist = clip(ref + rint(N(0,16)), 0, 1023)"),
    3: Workload(3, "3840x2160 12-bit", 3840, 2160, 32, 12,
                "ref and dist independent uniform 0..4095 (full-range noise)"),
    4: Workload(4, "1920x1080 16-bit bright", 1920, 1080, 40, 16,
                "ref and dist independent uniform 56000..64000"),
    5: Workload(5, "3840x2160 16-bit", 3840, 2160, 32, 16,
                "ref uniform 60000..65535; dist = clip(ref + rint(N(0,512)), 0, 65535)"),
    6: Workload(6, "2560x1440 16-bit mixed", 2560, 1440, 64, 16,
                "per plane: a tenth of the positions (uniform(0,1) < 0.1) uniform 0..4095, "
                "the rest uniform 49152..65535; ref and dist drawn alike and independently"),
}


def _frame_pair(number: int, rng: np.random.Generator, w: int, h: int):
    if number == 1:
        ref = rng.integers(0, 255, size=(h, w), endpoint=True, dtype=np.int64)
        dist = np.clip(ref + np.rint(rng.normal(0.0, 8.0, size=(h, w))).astype(np.int64), 0, 255)
        return ref.astype(np.uint8), dist.astype(np.uint8)
    if number == 2:
        x = np.arange(w, dtype=np.float64)[None, :] / (w - 1)
        y = np.arange(h, dtype=np.float64)[:, None] / (h - 1)
        ramp = 1023.0 * (x + y) / 2.0
        ref = np.clip(np.rint(ramp + rng.normal(0.0, 40.0, size=(h, w))), 0, 1023).astype(np.int64)
        dist = np.clip(ref + np.rint(rng.normal(0.0, 16.0, size=(h, w))).astype(np.int64), 0, 1023)
        return ref.astype(np.uint16), dist.astype(np.uint16)
    if number == 3:
        ref = rng.integers(0, 4095, size=(h, w), endpoint=True, dtype=np.uint16)
        dist = rng.integers(0, 4095, size=(h, w), endpoint=True, dtype=np.uint16)
        return ref, dist
    if number == 4:
        ref = rng.integers(56000, 64000, size=(h, w), endpoint=True, dtype=np.uint16)
        dist = rng.integers(56000, 64000, size=(h, w), endpoint=True, dtype=np.uint16)
        return ref, dist
    if number == 5:
        ref = rng.integers(60000, 65535, size=(h, w), endpoint=True, dtype=np.int64)
        dist = np.clip(ref + np.rint(rng.normal(0.0, 512.0, size=(h, w))).astype(np.int64), 0, 65535)
        return ref.astype(np.uint16), dist.astype(np.uint16)
    if number == 6:
        out = []
        for _ in range(2):
            low = rng.random(size=(h, w)) < 0.1
            dark = rng.integers(0, 4095, size=(h, w), endpoint=True, dtype=np.uint16)
            bright = rng.integers(49152, 65535, size=(h, w), endpoint=True, dtype=np.uint16)
            out.append(np.where(low, dark, bright).astype(np.uint16))
        return out[0], out[1]
    raise ValueError(f"no workload {number}")


def generate(number: int, nframes: int | None = None, w: int | None = None, h: int | None = None):
    """Return ``(ref, dist)`` for a named workload.

    ``nframes``, ``w`` and ``h`` default to the workload's own; a smaller
    value draws the same recipe at another size (the first ``k`` frames at
    the workload's own size are the same whatever ``nframes`` is).
    """
    wl = WORKLOADS[number]
    nframes = wl.nframes if nframes is None else nframes
    w = wl.w if w is None else w
    h = wl.h if h is None else h
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    ref = np.empty((nframes, h, w), dtype=wl.dtype)
    dist = np.empty((nframes, h, w), dtype=wl.dtype)
    for f in range(nframes):
        ref[f], dist[f] = _frame_pair(number, rng, w, h)
    return ref, dist


CHROMA = {"420": (2, 2), "422": (2, 1), "444": (1, 1)}  # horizontal, vertical subsampling


def planar_yuv(number: int, chroma: str = "420", nframes: int | None = None):
    """Planar YUV frames of a workload: ``(ref, dist, planes)``.

    ``ref`` and ``dist`` are ``[nframes][frame_samples]`` arrays, each frame
    its Y plane then its U and V planes, row after row; ``planes`` lists
    ``(offset, w, h)`` of the three planes inside a frame.  Each plane is drawn
    with the workload's recipe at the plane's size, Y then U then V, frame
    after frame, from one generator seeded like the workload.
    """
    wl = WORKLOADS[number]
    nframes = wl.nframes if nframes is None else nframes
    sx, sy = CHROMA[chroma]
    cw, ch = -(-wl.w // sx), -(-wl.h // sy)
    planes = [(0, wl.w, wl.h), (wl.w * wl.h, cw, ch), (wl.w * wl.h + cw * ch, cw, ch)]
    frame = wl.w * wl.h + 2 * cw * ch
    rng = np.random.Generator(np.random.PCG64(wl.seed + 7000))
    ref = np.empty((nframes, frame), dtype=wl.dtype)
    dist = np.empty((nframes, frame), dtype=wl.dtype)
    for f in range(nframes):
        for off, pw, ph in planes:
            r, d = _frame_pair(number, rng, pw, ph)
            ref[f, off:off + pw * ph] = r.ravel()
            dist[f, off:off + pw * ph] = d.ravel()
    return ref, dist, planes


def uniform_planes(w: int, h: int, nframes: int, bpc: int, seed: int,
                   lo: int = 0, hi: int | None = None, container_max: bool = False):
    """Independent uniform ref and dist planes with values lo..hi.

    ``hi`` defaults to ``2**bpc - 1``.  With ``container_max`` the values span
    the whole container (0..255 or 0..65535) whatever ``bpc`` says: samples
    above ``2**bpc - 1`` are legal input and must be reduced like any other.
    """
    dtype = np.uint8 if bpc == 8 else np.uint16
    if container_max:
        hi = 255 if bpc == 8 else 65535
    elif hi is None:
        hi = (1 << bpc) - 1
    rng = np.random.Generator(np.random.PCG64(seed))
    ref = rng.integers(lo, hi, size=(nframes, h, w), endpoint=True, dtype=dtype)
    dist = rng.integers(lo, hi, size=(nframes, h, w), endpoint=True, dtype=dtype)
    return ref, dist


def past53_mixed(seed: int = 2053, w: int = 2560, h: int = 1440, nframes: int = 1):
    """16-bit frames with a tenth of the samples below 4096.

    Stand-in for the 2560x1440 frame past 2**53 units that the float_moment
    page measures.  A tenth of the positions, drawn at random, get uniform
    0..4095; the rest get uniform 49152..65535, bright enough that the sum of
    the float squares of one plane passes 2**53 units.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(2):
        low = rng.random(size=(nframes, h, w)) < 0.1
        dark = rng.integers(0, 4095, size=(nframes, h, w), endpoint=True, dtype=np.uint16)
        bright = rng.integers(49152, 65535, size=(nframes, h, w), endpoint=True, dtype=np.uint16)
        out.append(np.where(low, dark, bright).astype(np.uint16))
    return out[0], out[1]


def odd_dark_bright(seed: int = 4053, w: int = 3840, h: int = 2160, nframes: int = 1):
    """16-bit frames where a tenth of the samples are odd values 1..4095.

    The rest are uniform 49152..65535, so each plane's sum of float squares
    runs well past 2**54 units.  The squares of the dark samples are odd and
    exact; those of the bright ones are multiples of 2**8.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(2):
        low = rng.random(size=(nframes, h, w)) < 0.1
        dark = (2 * rng.integers(0, 2047, size=(nframes, h, w), endpoint=True) + 1).astype(np.uint16)
        bright = rng.integers(49152, 65535, size=(nframes, h, w), endpoint=True, dtype=np.uint16)
        out.append(np.where(low, dark, bright).astype(np.uint16))
    return out[0], out[1]


def past53_fullrange(seed: int = 3053, w: int = 3840, h: int = 2160, nframes: int = 1):
    """Independent full-range 16-bit noise (uniform 0..65535) in ref and dist."""
    return uniform_planes(w, h, nframes, 16, seed, 0, 65535)


def constant_pair(w: int, h: int, nframes: int, bpc: int, ref_value: int, dist_value: int):
    """Constant planes: every ref sample ``ref_value``, every dist sample ``dist_value``."""
    dtype = np.uint8 if bpc == 8 else np.uint16
    ref = np.full((nframes, h, w), ref_value, dtype=dtype)
    dist = np.full((nframes, h, w), dist_value, dtype=dtype)
    return ref, dist


def sha256(*arrays) -> str:
    """Digest of the raw bytes of the given arrays, in order."""
    m = hashlib.sha256()
    for a in arrays:
        m.update(np.ascontiguousarray(a).tobytes())
    return m.hexdigest()


# ------------------------------------------------------- float term buffers

HVS_4K_BLOCKS = (548, 308)  # 8x8 blocks at a step of 7 over 3840x2160: 10 802 176 terms


def hvs_like_terms(nblocks: int, nplanes: int = 1, seed: int = 1397) -> np.ndarray:
    """Seeded stand-in for the psnr_hvs CPU extractor's term buffers:
    ``[nplanes][nblocks * 64]`` float32, 64 terms per 8x8 block (row-major
    within the block, blocks in raster order), each the binary32 square of a
    masked coefficient error, most of them zero.

    The real terms come from a DCT and CSF and masking tables that are not
    available here; this draws their shape instead.  Per block, a scale
    (lognormal around 8) times a weight falling off with the coefficient's
    row + column (a synthetic stand-in for a contrast sensitivity curve)
    times |N(0, 1)| gives the error; a per-block threshold between 0.12 and
    0.9 of the scale (the plane's offset drawn in 0.12..0.3) masks it; the
    term is the float square of what is left.  A plane has 15 to 32 % nonzero
    terms, as the psnr_hvs page reports.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    r, c = np.meshgrid(np.arange(8), np.arange(8), indexing="ij")
    weight = (1.0 / (1.0 + 0.25 * (r + c))).astype(np.float32).ravel()
    out = np.empty((nplanes, nblocks * 64), dtype=np.float32)
    err = np.empty((nblocks, 64), dtype=np.float32)  # reused: fresh pages are slow to touch
    for p in range(nplanes):
        lo = rng.uniform(0.12, 0.3)
        scale = (np.exp(rng.normal(0.0, 1.0, nblocks)) * 8.0).astype(np.float32)
        mask = (scale * rng.uniform(lo, lo + 0.6, nblocks).astype(np.float32)).astype(np.float32)
        rng.standard_normal(dtype=np.float32, out=err)
        np.abs(err, out=err)
        err *= scale[:, None]
        err *= weight[None, :]
        err -= mask[:, None]
        np.maximum(err, np.float32(0), out=err)
        np.multiply(err, err, out=out[p].reshape(nblocks, 64))
    return out


def float_terms(n: int, kind: str, seed: int) -> np.ndarray:
    """Seeded float32 term buffers of ``n`` terms that stress a running float
    sum: ``"uniform"`` (0..1), ``"spread"`` (magnitudes over 2^-30..2^30),
    ``"tiny"`` (subnormals and the smallest normals), ``"ties"`` (small
    integers and halves after a large first term, so that many adds fall
    halfway between two floats), ``"stall"`` (a large first term, then terms
    below half its last place, which never move the sum), ``"ascending"``
    and ``"huge"`` (terms near the largest float, so that the sum overflows
    to infinity)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "uniform":
        t = rng.random(n, dtype=np.float32)
    elif kind == "spread":
        t = (rng.random(n) * 2.0 ** rng.integers(-30, 31, n)).astype(np.float32)
    elif kind == "tiny":
        bits = rng.integers(0, 1 << 24, n, dtype=np.uint32)
        t = bits.view(np.float32).copy()
    elif kind == "ties":
        t = (rng.integers(0, 8, n) * 0.5).astype(np.float32)
        t[0] = np.float32(2.0 ** 22)
    elif kind == "stall":
        t = (rng.random(n) * 0.49).astype(np.float32)
        t[0] = np.float32(2.0 ** 24)
    elif kind == "ascending":
        t = np.sort(rng.random(n).astype(np.float32) * np.float32(1000.0))
    elif kind == "huge":
        t = (rng.random(n) * 1.0e37 + 1.0e37).astype(np.float32)
    else:
        raise ValueError(kind)
    return t.astype(np.float32)
