"""Pins that tie the oracle to facts other than itself.

Every pin takes an implementation object with four members --
``seq(ref, dist, bpc) -> [F][5] float64`` (the CPU's sequential double sums),
``exact(ref, dist) -> [F][5] int`` (exact integer sums),
``q(n) -> int`` (the float square of n as an integer) and
``bound(pixels, e, bpc) -> float`` -- and returns a list of failure strings
(empty: the pin holds).  The real oracle must pass all of them; each planted
mistake (tests/test_oracle_mutants.py) must fail at least one.

What the pins rest on:
  * IEEE 754 binary32 arithmetic as numpy performs it on the host (products
    and int-to-float conversions round to nearest even);
  * closed forms (identical planes, constant planes, constant differences);
  * a textbook routine (numpy.mean);
  * brute force on tiny planes, where every output is checked against the
    exact integer sum scaled by the unit;
  * the numbers the pages print (tests/golden/page_facts.json).
"""

from __future__ import annotations

import functools
import json
import math
import os

import numpy as np

import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
UNIT_POWER = (2, 1, 1, 2, 2)
TWO53 = 1 << 53


def page_facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return {x["id"]: x for x in json.load(f)["facts"]}


def _dtype(bpc):
    return np.uint8 if bpc == 8 else np.uint16


def _scaled_exact(exact_row, bpc):
    s = 1 << (bpc - 8)
    return [float(int(v)) / float(s ** p) for v, p in zip(exact_row, UNIT_POWER)]


# ---------------------------------------------------------------- the float square

def pin_q_matches_binary32_product(impl):
    """q(n) equals numpy's binary32 product n*n, for every n in 0..65535."""
    n = np.arange(1 << 16, dtype=np.int64)
    f = n.astype(np.float32)
    want = (f * f).astype(np.int64)
    got = np.array([impl.q(int(v)) for v in n], dtype=np.int64)
    bad = np.nonzero(got != want)[0]
    return [f"q({int(bad[0])}) = {int(got[bad[0]])}, binary32 product gives {int(want[bad[0]])}"
            f" ({bad.size} values differ)"] if bad.size else []


def pin_q_tie_cases(impl):
    """Hand-worked ties: 4097^2 = 2^24 + 8193 lies halfway between 16785408 and
    16785410 and goes to the even significand; 65535^2 = 4294836225 rounds
    down to 4294836224, an integer below 2^32 as the float_moment page says."""
    fails = []
    for n, want in ((4097, 16785408), (65535, 4294836224), (4096, 16777216), (4095, 16769025)):
        if impl.q(n) != want:
            fails.append(f"q({n}) = {impl.q(n)}, want {want}")
    return fails


# ---------------------------------------------------------------- closed forms

def pin_identical_planes(impl):
    """Identical planes have zero noise."""
    fails = []
    for bpc in (8, 10, 16):
        ref, _ = synth.uniform_planes(17, 9, 2, bpc, seed=11 + bpc, container_max=True)
        s = impl.seq(ref, ref.copy(), bpc)
        e = impl.exact(ref, ref.copy())
        if np.any(s[:, 0] != 0.0) or any(int(v) != 0 for v in e[:, 0]):
            fails.append(f"bpc {bpc}: noise of identical planes is not 0")
    return fails


def pin_constant_difference(impl):
    """A constant difference d gives noise w*h*d^2/scaler^2 for |d| <= 4096
    (d^2 <= 2^24 is exact in binary32), and w*h*q(d)/scaler^2 beyond."""
    fails = []
    w, h = 13, 7
    cases = [(8, 200, 199), (8, 0, 255), (10, 1023, 0), (12, 4095, 0), (16, 4096, 0),
             (16, 10, 4106), (16, 4097, 0), (16, 65535, 0), (14, 0, 9000)]
    for bpc, a, b in cases:
        ref, dist = synth.constant_pair(w, h, 1, bpc, a, b)
        d = abs(a - b)
        sq = d * d if d <= 4096 else {4097: 16785408, 65535: 4294836224, 9000: 81000000}[d]
        s2 = float((1 << (bpc - 8)) ** 2)
        want_seq = w * h * sq / s2
        got_seq = float(impl.seq(ref, dist, bpc)[0, 0])
        got_exact = int(impl.exact(ref, dist)[0, 0])
        if got_seq != want_seq:
            fails.append(f"bpc {bpc} d {d}: seq noise {got_seq!r} want {want_seq!r}")
        if got_exact != w * h * sq:
            fails.append(f"bpc {bpc} d {d}: exact noise {got_exact} want {w * h * sq}")
    return fails


def pin_constant_plane_moments(impl):
    """A constant plane c gives sum = w*h*c and sum of squares = w*h*q(c)."""
    fails = []
    w, h = 11, 5
    for bpc, c, sq in ((8, 255, 65025), (10, 777, 603729), (16, 65535, 4294836224),
                       (16, 40000, 1600000000), (12, 3, 9)):
        ref, dist = synth.constant_pair(w, h, 1, bpc, c, 0)
        s = float(1 << (bpc - 8))
        got = impl.seq(ref, dist, bpc)[0]
        ex = impl.exact(ref, dist)[0]
        if got[1] != w * h * c / s or got[2] != 0.0:
            fails.append(f"bpc {bpc} c {c}: first moments {got[1]!r}, {got[2]!r}")
        if got[3] != w * h * sq / (s * s) or got[4] != 0.0:
            fails.append(f"bpc {bpc} c {c}: second moments {got[3]!r}, {got[4]!r}")
        if int(ex[1]) != w * h * c or int(ex[3]) != w * h * sq or int(ex[2]) != 0 or int(ex[4]) != 0:
            fails.append(f"bpc {bpc} c {c}: exact moments {list(map(int, ex))}")
    return fails


def pin_first_moment_is_numpy_mean(impl):
    """The mean (first moment) equals numpy.mean of the samples over the scaler.

    Below 2^53 units every partial sum is exact whatever the order, so the
    CPU's sequential double and numpy's pairwise sum agree bit for bit."""
    fails = []
    for bpc, (w, h) in ((8, (33, 21)), (10, (64, 40)), (16, (50, 50))):
        ref, dist = synth.uniform_planes(w, h, 2, bpc, seed=100 + bpc, container_max=True)
        s = float(1 << (bpc - 8))
        got = impl.seq(ref, dist, bpc)
        for f in range(2):
            for k, plane in ((1, ref[f]), (2, dist[f])):
                mean = float(np.mean(plane.astype(np.float64) / s))
                if got[f, k] / (w * h) != mean:
                    fails.append(f"bpc {bpc} frame {f} output {k}: {got[f, k] / (w * h)!r} != {mean!r}")
    return fails


def pin_symmetry(impl):
    """Swapping ref and dist leaves the noise and swaps the moments."""
    ref, dist = synth.uniform_planes(19, 13, 1, 16, seed=7, container_max=True)
    a = impl.seq(ref, dist, 16)[0]
    b = impl.seq(dist, ref, 16)[0]
    if a[0] != b[0] or a[1] != b[2] or a[2] != b[1] or a[3] != b[4] or a[4] != b[3]:
        return ["seq is not symmetric under swapping ref and dist"]
    ea = [int(v) for v in impl.exact(ref, dist)[0]]
    eb = [int(v) for v in impl.exact(dist, ref)[0]]
    if ea[0] != eb[0] or ea[1] != eb[2] or ea[3] != eb[4]:
        return ["exact is not symmetric under swapping ref and dist"]
    return []


# ---------------------------------------------------------------- brute force

def _tiny_cases():
    rng = np.random.Generator(np.random.PCG64(424242))
    for bpc in range(8, 17):
        top = 255 if bpc == 8 else 65535
        for h in (1, 2, 3, 8):
            for w in (1, 2, 5, 8):
                ref = rng.integers(0, top, size=(2, h, w), endpoint=True).astype(_dtype(bpc))
                dist = rng.integers(0, top, size=(2, h, w), endpoint=True).astype(_dtype(bpc))
                yield bpc, ref, dist
        # adversarial values: extremes, ties, and values in the real range
        vals = np.array([0, 1, top, top - 1] + ([4095, 4096, 4097, 46341, 65535 - 4097]
                                                 if bpc > 8 else [128, 127]), dtype=np.int64)
        ref = np.resize(vals, (1, 3, vals.size)).astype(_dtype(bpc))
        dist = np.roll(ref, 1, axis=2)
        yield bpc, ref, dist


def pin_seq_equals_exact_tiny(impl):
    """Brute force on tiny planes (1x1 .. 8x8, bpc 8..16, values across the
    whole container): below 2^53 the CPU's doubles equal the exact integer
    sums scaled by the unit, output by output and frame by frame."""
    fails = []
    for bpc, ref, dist in _tiny_cases():
        s = impl.seq(ref, dist, bpc)
        e = impl.exact(ref, dist)
        for f in range(ref.shape[0]):
            brute = _brute_force_frame(ref[f], dist[f])
            if [int(v) for v in e[f]] != brute:
                fails.append(f"bpc {bpc} {ref.shape}: exact {list(map(int, e[f]))} != brute force {brute}")
            if list(s[f]) != _scaled_exact(brute, bpc):
                fails.append(f"bpc {bpc} {ref.shape}: seq {list(s[f])} != exact/unit")
        if len(fails) > 4:
            break
    return fails


def _brute_force_frame(ref, dist):
    """Per-sample Python loop with numpy's binary32 product as the square."""
    n = r1 = d1 = r2 = d2 = 0
    for a, b in zip(ref.ravel().tolist(), dist.ravel().tolist()):
        fa, fb = np.float32(a), np.float32(b)
        diff = np.float32(fa - fb)
        n += int(np.float32(diff * diff))
        r1 += a
        d1 += b
        r2 += int(np.float32(fa * fa))
        d2 += int(np.float32(fb * fb))
    return [n, r1, d1, r2, d2]


def pin_seq_equals_exact_discriminating(impl):
    """Frames where plausible shortcuts break: full-range noise at 8..16 bits
    (large block sums), bright 16-bit content (every square rounded), tie
    values, three frames in a batch (each frame starts from zero)."""
    fails = []
    cases = []
    for bpc in (8, 10, 12, 16):
        cases.append((bpc,) + synth.uniform_planes(48, 40, 3, bpc, seed=500 + bpc))
    cases.append((16,) + synth.uniform_planes(48, 40, 2, 16, seed=77, lo=56000, hi=64000))
    cases.append((13,) + synth.uniform_planes(32, 32, 2, 13, seed=78, container_max=True))
    ties = np.full((2, 16, 16), 4097, dtype=np.uint16)
    ties[1, ::2] = 46341
    cases.append((16, ties, np.zeros_like(ties)))
    for bpc, ref, dist in cases:
        s = impl.seq(ref, dist, bpc)
        e = impl.exact(ref, dist)
        for f in range(ref.shape[0]):
            brute = _brute_force_frame(ref[f], dist[f]) if ref[f].size <= 2048 else None
            ex = [int(v) for v in e[f]]
            if brute is not None and ex != brute:
                fails.append(f"bpc {bpc} frame {f}: exact {ex} != brute force {brute}")
            if list(s[f]) != _scaled_exact(ex, bpc):
                fails.append(f"bpc {bpc} frame {f}: seq {list(s[f])} != exact/unit {_scaled_exact(ex, bpc)}")
    return fails


def pin_block_facts(impl):
    """8-bit worst case (255 against 0): every square is below 2^16 and every
    16x16 block of 256 squares below 2^24; at 12 bits (4095 against 0) every
    block is below 2^32 [float_psnr page, Context and Decision]."""
    fails = []
    facts = page_facts()
    for bpc, top, key in ((8, 255, "block_8bit"), (12, 4095, "block_12bit_u32")):
        ref, dist = synth.constant_pair(16, 16, 1, bpc, top, 0)
        block = int(impl.exact(ref, dist)[0, 0])
        if block != 256 * top * top:
            fails.append(f"bpc {bpc}: block of 256 worst squares {block}")
        if not block < (1 << facts[key]["block_below_log2"]):
            fails.append(f"bpc {bpc}: block {block} not below 2^{facts[key]['block_below_log2']}")
    if not impl.q(255) < (1 << facts["block_8bit"]["square_below_log2"]):
        fails.append("8-bit square not below 2^16")
    if not impl.q(65535) < (1 << facts["square_16bit_below_2_32"]["below_log2"]):
        fails.append("16-bit square not below 2^32")
    return fails


# ---------------------------------------------------------------- past 2^53

def _mean_distance(impl, ref, dist, bpc):
    """Largest distance, over the two second moments (and the noise), between
    the CPU's mean and the exact mean; plus the binade e of the largest sum."""
    h, w = ref.shape[-2:]
    s = impl.seq(ref, dist, bpc)[0]
    e = [int(v) for v in impl.exact(ref, dist)[0]]
    scale = float((1 << (bpc - 8)) ** 2)
    out = []
    for k in (0, 3, 4):
        cpu = s[k] / (w * h)
        exact = (float(e[k]) / scale) / (w * h)
        out.append((abs(cpu - exact), e[k].bit_length() - 1, e[k]))
    return out


def pin_past53(impl):
    """Past 2^53 units the CPU's second moments stay within the page's bound of
    the exact ones; the page's three measured frames have e = 53, 53 and 0
    distance above 60000 [float_moment page, Decision and Consequences]."""
    fails = []
    facts = page_facts()
    mixed = synth.past53_mixed(w=2560, h=1440)
    full = synth.past53_fullrange(w=3840, h=2160)
    bright = synth.uniform_planes(3840, 2160, 1, 16, seed=61, lo=60001, hi=65535)
    for name, (ref, dist), fact in (("mixed 2560x1440", mixed, facts["bound_1440p"]),
                                    ("full-range 3840x2160", full, facts["bound_4k_noise"])):
        d = _mean_distance(impl, ref[0:1], dist[0:1], 16)
        for dist_k, e_k, sum_k in d[1:]:
            if sum_k < TWO53:
                fails.append(f"{name}: the second-moment sum {sum_k} does not pass 2^53")
                continue
            if e_k != fact["e"]:
                fails.append(f"{name}: binade {e_k}, the page's frame has {fact['e']}")
            b = impl.bound(ref.shape[-1] * ref.shape[-2], e_k, 16)
            if dist_k > b:
                fails.append(f"{name}: distance {dist_k} above bound {b}")
        if max(x[0] for x in d[1:]) == 0.0:
            fails.append(f"{name}: no rounding at all past 2^53 (expected a nonzero distance)")
    d = _mean_distance(impl, bright[0][0:1], bright[1][0:1], 16)
    for dist_k, e_k, sum_k in d[1:]:
        if sum_k < TWO53 or dist_k != facts["zero_above_60000"]["measured"]:
            fails.append(f"above 60000: distance {dist_k} (sum {sum_k}); the page measures 0")
    return fails


def pin_bound_printed_values(impl):
    """The bound reproduces the values the float_moment page prints."""
    fails = []
    for key in ("bound_4k_peak", "bound_4k_noise", "bound_1440p"):
        f = page_facts()[key]
        got = impl.bound(f["pixels"], f["e"], f["bpc"])
        if float(f"{got:.{f['digits'] - 1}e}") != f["bound"]:
            fails.append(f"{key}: bound {got:.3e}, page prints {f['bound']}")
    return fails


def pin_exact_range_facts(impl):
    """2^21 pixels and the 16-bit PSNR exact-range MSE the pages print."""
    fails = []
    facts = page_facts()
    f = facts["exact_range_pixels"]
    if f["w"] * f["h"] != f["pixels"] or not f["pixels"] <= f["pixels_limit"] == 1 << 21:
        fails.append("1920x1080 is not within 2^21 pixels")
    # largest 1080p frame of largest terms (65535 against 0): exact sum below 2^53
    if f["pixels"] * impl.q(65535) >= TWO53:
        fails.append("a 1920x1080 frame of largest terms reaches 2^53 units")
    for key in ("psnr_exact_range_4k", "psnr_exact_range_1080p"):
        g = facts[key]
        mse = 2.0 ** 37 / (g["w"] * g["h"])
        if float(f"{mse:.{g['digits'] - 1}e}") != float(f"{g['mse']:.{g['digits'] - 1}e}"):
            fails.append(f"{key}: 2^37/(w*h) = {mse}, page prints {g['mse']}")
    g = facts["psnr_exact_range_4k"]
    p = 65535 / 256
    if not 10 * math.log10(p * p / (2.0 ** 37 / (g["w"] * g["h"]))) < g["psnr_below_db"]:
        fails.append("PSNR at the 4K limit is not below 6 dB")
    # up to 12 bits: 2^25 pixels (the largest frame the library accepts) of
    # 12-bit squares need at most 49 bits
    if (33554432 * 4095 * 4095).bit_length() > facts["sum_49_bits_12bit"]["bits"]:
        fails.append("12-bit noise of 2^25 pixels needs more than 49 bits")
    return fails


# ------------------------------------------------ the CPU's order past 2^53

def rn53(n: int) -> int:
    """Nonnegative integer ``n`` rounded to 53 significant bits, ties to even.

    binary64 keeps a 53-bit significand and rounds to nearest, ties to even
    (IEEE 754's default).  Integers up to 2^53 fit as they are.  Otherwise,
    with k = bitlength(n) - 53 and n = Q*2^k + r, keep Q and add one when r
    is above half of 2^k, or exactly half and Q is odd.  Integers only.
    """
    k = n.bit_length() - 53
    if k <= 0:
        return n
    q = n >> k
    r = n - (q << k)
    half = 1 << (k - 1)
    if r > half or (r == half and (q & 1)):
        q += 1
    return q << k


def binary64_running_sum(terms) -> int:
    """The value a binary64 accumulator holds after adding the nonnegative
    integer ``terms`` to zero one at a time, in the given order:
    S <- rn53(S + t) at every add.

    Every partial sum up to 2^53 is exact, so the prefix up to the last such
    partial sum is taken with an exact int64 running total; the adds from
    there on are done one by one.
    """
    terms = np.asarray(terms, dtype=np.int64).ravel()
    if terms.size == 0:
        return 0
    prefix = np.cumsum(terms)  # exact: below 2^25 * 2^32
    past = np.nonzero(prefix > TWO53)[0]
    if past.size == 0:
        return int(prefix[-1])
    i0 = int(past[0])
    s = int(prefix[i0 - 1]) if i0 else 0
    for t in terms[i0:].tolist():
        s = rn53(s + t)
    return s


def _binary32_square_units(x):
    """The binary32 product x*x of each stored integer x, read back as an
    integer (numpy's float32 multiply rounds to nearest even)."""
    f = np.asarray(x).astype(np.float32)
    return (f * f).astype(np.int64)


@functools.lru_cache(maxsize=None)
def _past53_frames():
    """The three frames past 2^53 units, and the CPU's five sums of each as
    integers in units, emulated in raster order (rows top to bottom, columns
    left to right) with ``binary64_running_sum``."""
    frames = {
        "mixed 2560x1440": synth.past53_mixed(w=2560, h=1440),
        "full-range 3840x2160": synth.past53_fullrange(w=3840, h=2160),
        "odd dark, bright 3840x2160": synth.odd_dark_bright(w=3840, h=2160),
    }
    out = {}
    for name, (ref, dist) in frames.items():
        r = ref[0].astype(np.int64).ravel()
        d = dist[0].astype(np.int64).ravel()
        terms = (_binary32_square_units(np.abs(r - d)), r, d,
                 _binary32_square_units(r), _binary32_square_units(d))
        out[name] = (ref[0:1], dist[0:1], [binary64_running_sum(t) for t in terms])
    return out


def pin_past53_raster_order(impl):
    """Past 2^53 units the CPU's running double rounds at every add, in the
    order it visits the samples; no other order gives the same bits [float_psnr
    page, Consequences: past 2^53 the CPU's sum rounds in sequence; float_moment
    page, Alternatives: reproducing that sequence of roundings].  The CPU visits
    rows top to bottom and each row left to right [float_psnr page, Context].
    O1 must equal an integer-only emulation of S <- RN53(S + t) in that order,
    bit for bit, on frames whose second moments pass 2^53 (ties at every binade,
    full-range noise, and odd dark squares under bright ones past 2^54)."""
    fails = []
    for name, (ref, dist, want) in _past53_frames().items():
        got = impl.seq(ref, dist, 16)[0]
        if not any(w > TWO53 for w in want):
            fails.append(f"{name}: no sum passes 2^53")
        for k in range(5):
            units = float(got[k]) * float(256 ** UNIT_POWER[k])  # exact: a power of two
            if units != float(want[k]) or int(units) != want[k]:
                fails.append(f"{name}: output {k} is {int(units)} units, the sequential "
                             f"binary64 sum in raster order is {want[k]}")
    return fails


def pin_past53_bound_below_16_bits(impl):
    """The bound's reading for 13..15 bits.  The pages state the bound at 16
    bits only [float_moment page, Decision].  With the same stored integers, a
    depth of bpc scales every CPU term, partial sum and mean by
    2^(2*(16 - bpc)) (exact: a power of two), so the CPU's sums at bpc are the
    16-bit sums scaled, and the bound must scale the same way.  Checked on the
    mixed frame (values up to 65535 in the container, which the library
    accepts at any depth): O1 at 13, 14 and 15 bits equals the raster-order
    emulation scaled; the CPU mean lies within the bound of the exact mean;
    and the bound is the 16-bit bound times 2^(2*(16 - bpc))."""
    fails = []
    ref, dist, want = _past53_frames()["mixed 2560x1440"]
    exact = [int(v) for v in impl.exact(ref, dist)[0]]
    pixels = ref.shape[-1] * ref.shape[-2]
    for bpc in (13, 14, 15):
        s = 1 << (bpc - 8)
        got = impl.seq(ref, dist, bpc)[0]
        for k in (0, 3, 4):
            unit = float(s ** UNIT_POWER[k])
            if float(got[k]) * unit != float(want[k]):
                fails.append(f"bpc {bpc} output {k}: {float(got[k]) * unit} units, "
                             f"emulation {want[k]}")
            if exact[k] <= TWO53:
                continue
            e = max(binade_int(exact[k]), binade_int(want[k]))
            b = impl.bound(pixels, e, bpc)
            cpu_mean = float(got[k]) / pixels
            exact_mean = (float(exact[k]) / unit) / pixels
            if abs(cpu_mean - exact_mean) > b:
                fails.append(f"bpc {bpc} output {k}: distance {abs(cpu_mean - exact_mean)} > bound {b}")
            b16 = impl.bound(pixels, e, 16)
            if b != b16 * 2.0 ** (2 * (16 - bpc)):
                fails.append(f"bpc {bpc}: bound {b} is not the 16-bit bound {b16} times "
                             f"2^{2 * (16 - bpc)}")
    return fails


def binade_int(n: int) -> int:
    """e with 2^e <= n < 2^(e+1), for an integer n > 0."""
    return n.bit_length() - 1


ALL_PINS = [
    pin_q_matches_binary32_product,
    pin_q_tie_cases,
    pin_identical_planes,
    pin_constant_difference,
    pin_constant_plane_moments,
    pin_first_moment_is_numpy_mean,
    pin_symmetry,
    pin_seq_equals_exact_tiny,
    pin_seq_equals_exact_discriminating,
    pin_block_facts,
    pin_past53,
    pin_bound_printed_values,
    pin_exact_range_facts,
    pin_past53_raster_order,
    pin_past53_bound_below_16_bits,
]

# Pins that take seconds (frames of millions of samples); run them last.
SLOW_PINS = (pin_past53, pin_past53_raster_order, pin_past53_bound_below_16_bits)


class RealOracle:
    """The oracle as shipped."""

    def __init__(self):
        import oracle
        self._o = oracle

    def seq(self, ref, dist, bpc):
        return self._o.seq_batch_sums(ref, dist, bpc)

    def exact(self, ref, dist):
        return self._o.exact_batch_sums(ref, dist)

    def q(self, n):
        return self._o.q_int(n)

    def bound(self, pixels, e, bpc):
        return self._o.past53_bound(pixels, e, bpc)


def run_all(impl, pins=None):
    """{pin name: failures} for every pin that fails."""
    out = {}
    for pin in pins or ALL_PINS:
        fails = pin(impl)
        if fails:
            out[pin.__name__] = fails
    return out
