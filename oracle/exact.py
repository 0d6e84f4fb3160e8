"""TEST INFRASTRUCTURE ONLY: exact-integer oracle, comparison bound, conclusions.

Only the tests, the smoke check and the bench's cpu_baseline leg may use this
module; no product code path does.  It shares no code with the HIP library.

Sources (web pages, cited by title and section):

* [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as integers
  and returns the CPU's score bit for bit" -- Context, Decision, Consequences.
* [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU adds,
  and is bit-identical while the CPU's own sum is exact" -- Context, Decision.

What is computed here, and why it is the CPU's result:

* q(n) is the float square of a sample (or of a sample difference) expressed
  as an integer in units of 1/scaler^2.  Scaling by a power of two does not
  change which bits a float product drops [MOMENT, Decision], so q(n) is the
  integer n*n rounded to a 24-bit significand, ties to even (binary32's
  significand width and default rounding).  ``rne24`` writes that rounding
  out with integers only, from the IEEE 754 definition of round-to-nearest-
  even; it uses no floating point.
* The five exact sums of a frame: N = sum q(ref - dist) (units 1/s^2),
  S1r = sum ref, S1d = sum dist (units 1/s), S2r = sum q(ref),
  S2d = sum q(dist) (units 1/s^2).  Every CPU term is a multiple of its unit,
  so the CPU's double sum equals this integer (times the unit) while it stays
  below 2^53 units [PSNR, Context; MOMENT, Decision].
* Past 2^53 units the CPU's running double rounds; the distance between its
  mean and the exact mean is bounded by ``past53_bound`` [MOMENT, Decision].
"""

from __future__ import annotations

import math
from functools import lru_cache

import numpy as np

TWO53 = 1 << 53

# Output order shared by every sum tuple in this module.
NOISE, REF_SUM, DIST_SUM, REF_SQ, DIST_SQ = range(5)
# Power of the scaler in each output's unit: squares are in 1/s^2, samples in 1/s.
UNIT_POWER = (2, 1, 1, 2, 2)


def rne24(n: int) -> int:
    """Nonnegative integer ``n`` rounded to 24 significant bits, ties to even.

    Below 2^24 every integer already fits and is returned unchanged.
    Otherwise with k = bitlength(n) - 24, n = Q*2^k + r: keep Q, add one
    when r is above half of 2^k, or exactly half and Q is odd.
    """
    if n < 0:
        raise ValueError("rne24 takes a nonnegative integer")
    if n < (1 << 24):
        return n
    k = n.bit_length() - 24
    q, r = divmod(n, 1 << k)
    half = 1 << (k - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return q << k


def q_int(n: int) -> int:
    """The float square of the integer n as an integer: rne24(n*n)."""
    return rne24(n * n)


@lru_cache(maxsize=1)
def q_table() -> np.ndarray:
    """q(n) for n = 0..65535 as int64, built with ``q_int`` (integers only)."""
    return np.array([q_int(n) for n in range(1 << 16)], dtype=np.int64)


def scaler(bpc: int) -> int:
    """scaler = 2^(bpc - 8) [PSNR, Context]."""
    if not 8 <= bpc <= 16:
        raise ValueError("bpc must be 8..16")
    return 1 << (bpc - 8)


def exact_frame_sums(ref: np.ndarray, dist: np.ndarray) -> tuple:
    """Exact (N, S1r, S1d, S2r, S2d) of one frame as Python ints.

    ``ref`` and ``dist`` hold the stored sample integers (any shape, same
    shape).  The sums are taken in int64, which is exact here: a frame has at
    most 2^25 samples and a term is below 2^32.
    """
    r = np.asarray(ref).astype(np.int64).ravel()
    d = np.asarray(dist).astype(np.int64).ravel()
    if r.shape != d.shape:
        raise ValueError("ref and dist differ in shape")
    if r.size and (r.min() < 0 or r.max() > 65535 or d.min() < 0 or d.max() > 65535):
        raise ValueError("samples must be 0..65535")
    t = q_table()
    return (int(t[np.abs(r - d)].sum()), int(r.sum()), int(d.sum()),
            int(t[r].sum()), int(t[d].sum()))


def exact_batch_sums(ref: np.ndarray, dist: np.ndarray) -> np.ndarray:
    """[nframes][5] int64 exact sums for a ``[nframes][h][w]`` batch."""
    return np.array([exact_frame_sums(ref[f], dist[f]) for f in range(ref.shape[0])],
                    dtype=np.int64).reshape(-1, 5)


def binade(x: float | int) -> int:
    """e with 2^e <= x < 2^(e+1), for x > 0."""
    if isinstance(x, int):
        return x.bit_length() - 1
    m, e = math.frexp(x)
    return e - 1


def past53_bound(pixels: int, e: int, bpc: int = 16) -> float:
    """Largest distance between the CPU's mean and the exact mean past 2^53 units.

    [MOMENT, Decision], for 16 bits: the first 2^21 adds of terms below 2^32
    units are exact; each of the remaining pixels - 2^21 adds, and the exact
    sum's one rounding to double, moves the value by at most half an ulp,
    2^(e-53) units; a unit of a second moment is 2^-16 divided by the pixel
    count; the two final divisions add at most 2^-37, which gives
    (pixels - 2^21 + 1)/pixels * 2^(e-69) + 2^-37.

    Reading for 13..15 bits (the pages treat only 16): the same argument
    with a unit of 1/scaler^2 = 2^-2(bpc-8), and the division term scaled
    with the largest mean, 2^32 units, i.e. 2^-37 * 2^(32 - 2*(bpc-8)) / 2^16.
    At bpc = 16 both reduce to the page's expression.
    """
    unit_exp = 2 * (bpc - 8)
    return ((pixels - (1 << 21) + 1) / pixels * 2.0 ** (e - 53 - unit_exp)
            + 2.0 ** (-37 + 16 - unit_exp))


def peak(bpc: int) -> float:
    """Largest sample on the 8-bit scale, (2^bpc - 1) / scaler.

    Reading: the pages print no PSNR formula; the mean squared error is on
    the 8-bit scale [PSNR, Consequences], so the peak is taken on that scale.
    """
    return ((1 << bpc) - 1) / scaler(bpc)


def psnr_db(mse: float, bpc: int, psnr_max: float = 0.0) -> float:
    """10*log10(peak^2/mse), capped at psnr_max when psnr_max > 0.

    mse == 0 gives psnr_max, or +inf without a cap.  (Textbook PSNR; the
    cap's existence follows from the tool's uncapped option [PSNR,
    Consequences]; its value is the caller's.)
    """
    if mse == 0.0:
        return psnr_max if psnr_max > 0 else math.inf
    p = peak(bpc)
    v = 10.0 * math.log10(p * p / mse)
    return min(v, psnr_max) if psnr_max > 0 else v


def conclude_from_doubles(sums5, w: int, h: int):
    """CPU conclusion from the five 8-bit-scale doubles: each over w*h.

    Returns (mse, ref_mean, dist_mean, ref_mean_sq, dist_mean_sq).
    """
    n = float(w * h)
    return tuple(float(s) / n for s in sums5)


def conclude_from_ints(sums5, w: int, h: int, bpc: int):
    """Conclusion from exact integer sums: to double (one rounding), then the
    two divisions, by scaler^k (exact) and by w*h [MOMENT, Decision; PSNR,
    Decision].  Python's int-to-float conversion rounds to nearest even."""
    s = scaler(bpc)
    n = float(w * h)
    return tuple((float(int(v)) / float(s ** p)) / n for v, p in zip(sums5, UNIT_POWER))


def acceptance(device5, o1_5, o2_5, w: int, h: int, bpc: int):
    """Compare device integer sums with the two oracles, output by output.

    Returns a list of (output index, reason) for every failed rule; empty
    means the device result is accepted.

    1. The device integer equals the exact integer, always.
    2. Where the exact sum is below 2^53 units the CPU's double equals it
       after scaling, and the concluded means are bitwise equal.
    3. Otherwise the concluded means differ by at most ``past53_bound``.
    """
    fails = []
    s = scaler(bpc)
    pixels = w * h
    dev_mean = conclude_from_ints(device5, w, h, bpc)
    cpu_mean = conclude_from_doubles(o1_5, w, h)
    for k in range(5):
        dev = int(device5[k])
        exact = int(o2_5[k])
        if dev != exact:
            fails.append((k, f"device {dev} != exact {exact}"))
            continue
        if exact < TWO53:
            if float(exact) / float(s ** UNIT_POWER[k]) != float(o1_5[k]):
                fails.append((k, "CPU double is not the exact sum below 2^53"))
            if dev_mean[k] != cpu_mean[k]:
                fails.append((k, f"mean {dev_mean[k]!r} != CPU {cpu_mean[k]!r}"))
        else:
            cpu_units = float(o1_5[k]) * float(s ** UNIT_POWER[k])
            e = max(binade(exact), binade(cpu_units))
            b = past53_bound(pixels, e, bpc)
            if abs(dev_mean[k] - cpu_mean[k]) > b:
                fails.append((k, f"|{dev_mean[k]!r} - {cpu_mean[k]!r}| > bound {b}"))
    return fails
