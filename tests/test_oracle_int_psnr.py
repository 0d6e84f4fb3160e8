"""Pins of the integer psnr oracle (O3), and planted mistakes they catch (CPU).

Each pin holds O3 to something other than itself:

* a closed form: constant planes, noise = (a - b)^2 * w * h;
* brute force: pure-Python loops over tiny planes;
* O2, the independent float-square oracle: wherever |ref - dist| < 4096 the
  float square is exact, so O3's noise equals O2's noise (in 1/scaler^2);
* the worked tie of the float_moment page (MOMENT, Decision): 4097^2 =
  2^24 + 8193 rounds to 16 785 408 as a float square, so a plane whose
  differences are all 4097 has an integer noise one unit per sample above
  O2's;
* textbook PSNR values: 8-bit mse 1 gives 20*log10(255) dB; the cap and the
  uncapped mse = 0 case.

Sources: "ADR-1440: float_psnr_hip adds its squared differences as integers
and returns the CPU's score bit for bit" (Alternatives: the integer psnr twin
keeps one uint64 per frame); "ADR-1447: float_moment_hip adds the float
squares the CPU adds, and is bit-identical while the CPU's own sum is exact"
(Decision: the 4097 tie).
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import synth


class O3:
    noise = staticmethod(oracle.int_noise)
    psnr = staticmethod(oracle.int_psnr_db)


def _planes(rng, w, h, bpc, lo=0, hi=None):
    hi = (1 << bpc) - 1 if hi is None else hi
    dt = np.uint8 if bpc == 8 else np.uint16
    return (rng.integers(lo, hi, size=(h, w), endpoint=True).astype(dt),
            rng.integers(lo, hi, size=(h, w), endpoint=True).astype(dt))


def pin_constant(impl):
    for a, b, w, h in ((0, 0, 7, 3), (255, 0, 5, 5), (65535, 0, 64, 33), (1000, 4097 + 1000, 9, 2)):
        ref = np.full((h, w), a, dtype=np.uint16)
        dist = np.full((h, w), b, dtype=np.uint16)
        assert impl.noise(ref, dist) == (a - b) ** 2 * w * h


def pin_brute_force(impl):
    rng = np.random.default_rng(5)
    for bpc in (8, 10, 16):
        for w, h in ((1, 1), (3, 2), (8, 5)):
            ref, dist = _planes(rng, w, h, bpc)
            want = 0
            for y in range(h):
                for x in range(w):
                    e = int(ref[y, x]) - int(dist[y, x])
                    want += e * e
            assert impl.noise(ref, dist) == want


def pin_equals_float_noise_where_exact(impl):
    rng = np.random.default_rng(6)
    for bpc in (8, 10, 12):
        ref, dist = _planes(rng, 40, 17, bpc)
        assert impl.noise(ref, dist) == oracle.exact_frame_sums(ref, dist)[oracle.NOISE]
    # 16 bits with every difference below 4096
    ref, _ = _planes(rng, 40, 17, 16, lo=4096, hi=60000)
    dist = (ref.astype(np.int64) + rng.integers(-4095, 4095, size=ref.shape, endpoint=True)).astype(np.uint16)
    assert impl.noise(ref, dist) == oracle.exact_frame_sums(ref, dist)[oracle.NOISE]


def pin_page_tie(impl):
    ref = np.full((3, 5), 4097 + 100, dtype=np.uint16)
    dist = np.full((3, 5), 100, dtype=np.uint16)
    n = impl.noise(ref, dist)
    assert n == 15 * (2 ** 24 + 8193)
    assert n - oracle.exact_frame_sums(ref, dist)[oracle.NOISE] == 15


def pin_sign_and_order(impl):
    rng = np.random.default_rng(7)
    ref, dist = _planes(rng, 11, 6, 16)
    assert impl.noise(ref, dist) == impl.noise(dist, ref)
    assert impl.noise(ref, ref) == 0
    # the whole plane counts: the last row and column too
    bump = ref.copy()
    bump[-1, -1] ^= 1
    assert impl.noise(ref, bump) == 1


def pin_psnr_values(impl):
    # 8 bits, every difference 1: mse 1, psnr 20*log10(255)
    ref = np.full((4, 4), 11, dtype=np.uint8)
    dist = np.full((4, 4), 10, dtype=np.uint8)
    n = impl.noise(ref, dist)
    assert impl.psnr(n, 4, 4, 8) == pytest.approx(20 * math.log10(255), abs=1e-12)
    assert impl.psnr(n, 4, 4, 8) == 10 * math.log10(255.0 * 255.0 / 1.0)
    # 10 bits: mse 4 -> 10*log10(1023^2/4)
    assert impl.psnr(4 * 100, 10, 10, 10) == 10 * math.log10(1023.0 ** 2 / 4.0)
    # cap and mse 0
    assert impl.psnr(0, 10, 10, 10, 72.0) == 72.0
    assert math.isinf(impl.psnr(0, 10, 10, 10))
    assert impl.psnr(1, 1000, 1000, 16, 108.0) == 108.0  # the cap binds
    # the mse in double: a noise that needs 25 bits, over 3 samples
    n25 = (1 << 24) + 1
    assert impl.psnr(n25, 3, 1, 16) == 10 * math.log10(65535.0 ** 2 / (float(n25) / 3.0))
    # the mse division: noise to double once, then / (w*h)
    big = (1 << 53) + 1
    assert impl.psnr(big, 4096, 2048, 16) == 10 * math.log10(65535.0 ** 2 / (float(big) / (4096 * 2048)))


def pin_views(impl):
    """A region, a pitched plane and a subsampled chroma plane are the same
    function of the samples they select."""
    rng = np.random.default_rng(8)
    big_r, big_d = _planes(rng, 50, 30, 12)
    roi = (slice(3, 27), slice(5, 46))
    want = 0
    for y in range(3, 27):
        for x in range(5, 46):
            e = int(big_r[y, x]) - int(big_d[y, x])
            want += e * e
    assert impl.noise(big_r[roi], big_d[roi]) == want
    assert impl.noise(big_r[::2, ::2], big_d[::2, ::2]) == sum(
        (int(a) - int(b)) ** 2 for a, b in zip(big_r[::2, ::2].ravel(), big_d[::2, ::2].ravel()))


PINS = [pin_constant, pin_brute_force, pin_equals_float_noise_where_exact, pin_page_tie,
        pin_sign_and_order, pin_psnr_values, pin_views]


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin):
    pin(O3)


# ------------------------------------------------------------- planted mistakes
def _float_square_noise(ref, dist):
    e = np.abs(ref.astype(np.float32) - dist.astype(np.float32))
    return int((e * e).astype(np.float64).sum())


def _wrapping_noise(ref, dist):  # differences in the sample type: wraps below zero
    e = (ref - dist).astype(np.int64)
    return int((e * e).sum())


def _u32_noise(ref, dist):  # sum kept in 32 bits
    e = ref.astype(np.int64) - dist.astype(np.int64)
    return int((e * e).sum()) & 0xFFFFFFFF


def _dropped_last_row(ref, dist):
    e = ref[:-1].astype(np.int64) - dist[:-1].astype(np.int64)
    return int((e * e).sum())


def _8bit_scale_noise(ref, dist):  # float_psnr's unit mistaken for this one
    e = ref.astype(np.int64) - dist.astype(np.int64)
    return int((e * e).sum()) // 4


def _psnr_on_8bit_peak(noise, w, h, bpc, psnr_max=0.0):
    mse = float(noise) / float(w * h)
    if mse == 0.0:
        return psnr_max if psnr_max > 0 else math.inf
    v = 10.0 * math.log10(255.0 * 255.0 / mse)
    return min(v, psnr_max) if psnr_max > 0 else v


def _psnr_mse_in_float32(noise, w, h, bpc, psnr_max=0.0):
    mse = float(np.float32(noise) / np.float32(w * h))
    if mse == 0.0:
        return psnr_max if psnr_max > 0 else math.inf
    p = float((1 << bpc) - 1)
    v = 10.0 * math.log10(p * p / mse)
    return min(v, psnr_max) if psnr_max > 0 else v


def _psnr_no_cap(noise, w, h, bpc, psnr_max=0.0):
    return oracle.int_psnr_db(noise, w, h, bpc, 0.0)


MUTANTS = {
    "float squares": dict(noise=_float_square_noise),
    "wrapping difference": dict(noise=_wrapping_noise),
    "32-bit sum": dict(noise=_u32_noise),
    "dropped last row": dict(noise=_dropped_last_row),
    "8-bit scale": dict(noise=_8bit_scale_noise),
    "8-bit peak": dict(psnr=_psnr_on_8bit_peak),
    "float32 mse": dict(psnr=_psnr_mse_in_float32),
    "cap ignored": dict(psnr=_psnr_no_cap),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_caught(name):
    impl = type("Mutant", (O3,), {k: staticmethod(v) for k, v in MUTANTS[name].items()})
    caught = []
    for pin in PINS:
        try:
            pin(impl)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"mutant {name!r} passed every pin"


def test_batch_matches_frames():
    ref, dist = synth.uniform_planes(13, 7, 3, 16, seed=9, container_max=True)
    got = oracle.int_noise_batch(ref, dist)
    assert [int(v) for v in got] == [oracle.int_noise(ref[f], dist[f]) for f in range(3)]
