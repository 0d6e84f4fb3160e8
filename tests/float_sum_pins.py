"""Pins that tie the running float sum oracle (O4) to facts other than itself.

Every pin takes a function ``run(terms [nsums][n] float32) -> [nsums]
float32`` (the value of a binary32 accumulator after each buffer's terms are
added one by one from zero) and returns a list of failure strings (empty:
the pin holds).  The oracle must pass all of them; each planted mistake
(tests/test_float_sum_mutants.py) must fail at least one.

What the pins rest on:
  * an integer-only binary32 addition written from IEEE 754's definition
    (round to nearest, ties to even; subnormals; overflow to infinity),
    iterated in buffer order -- no floating point is used for it;
  * hand-worked sums around ties and at the ends of the number range;
  * closed forms (n ones; a sum that stalls);
  * a property of the definition: adding a zero leaves the sum as it was
    (the psnr_hvs page's Consequences).

Source: "ADR-1397: GPU psnr_hvs twins reproduce the CPU's running float sum
bit for bit" -- Context (one running float, each add's rounding depending on
the sum so far) and Decision (terms added one by one into a single float).
"""

from __future__ import annotations

import numpy as np

import synth

INF_BITS = 0x7F800000


def _units(bits: int) -> int:
    """A nonnegative finite binary32 value, given by its bit pattern, as an
    integer count of 2^-149 (the smallest subnormal)."""
    e = (bits >> 23) & 0xFF
    f = bits & 0x7FFFFF
    if e == 0xFF or bits >> 31:
        raise ValueError("nonnegative finite operands only")
    return f if e == 0 else (f | 0x800000) << (e - 1)


def _round_to_binary32(x: int) -> int:
    """The nonnegative integer x (units of 2^-149) rounded to a binary32
    value, ties to even, returned as a bit pattern.  Below 2^24 units every
    integer is representable (the subnormals and the lowest normal binade
    share the unit 2^-149); above, keep 24 significant bits."""
    k = x.bit_length() - 24
    if k > 0:
        q = x >> k
        r = x - (q << k)
        half = 1 << (k - 1)
        if r > half or (r == half and (q & 1)):
            q += 1
        x = q << k
    if x < (1 << 23):
        return x  # zero or subnormal: the bit pattern is the unit count
    s = x.bit_length() - 24  # x = M * 2^s with M of 24 bits
    exp_field = s + 1
    if exp_field >= 0xFF:
        return INF_BITS
    return (exp_field << 23) | ((x >> s) - (1 << 23))


def add_binary32(a_bits: int, b_bits: int) -> int:
    """IEEE 754 binary32 addition of two nonnegative operands (bit patterns),
    rounded to nearest, ties to even; infinity absorbs any finite operand."""
    if a_bits == INF_BITS or b_bits == INF_BITS:
        return INF_BITS
    # -0 adds like +0, and +0 + -0 is +0 under round to nearest
    a_bits = 0 if a_bits == 0x80000000 else a_bits
    b_bits = 0 if b_bits == 0x80000000 else b_bits
    return _round_to_binary32(_units(a_bits) + _units(b_bits))


def sequential_sum_bits(terms: np.ndarray) -> int:
    """The bit pattern of the running binary32 sum of ``terms`` (1-D), from
    +0, in order, with ``add_binary32``."""
    s = 0
    for b in np.ascontiguousarray(terms, dtype=np.float32).view(np.uint32).tolist():
        s = add_binary32(s, b)
    return s


def _bits(x) -> int:
    return int(np.asarray(x, dtype=np.float32).view(np.uint32))


# ---------------------------------------------------------------- the pins

def pin_matches_integer_emulation(run):
    """Bit for bit equal to the integer-only emulation on buffers of every
    kind: psnr_hvs-like terms, uniform, wide spread, subnormals, ties, a
    stalled sum, ascending terms, overflow to infinity."""
    fails = []
    bufs = [("hvs-like", synth.hvs_like_terms(1500, 2, seed=11))]
    for kind in ("uniform", "spread", "tiny", "ties", "stall", "ascending", "huge"):
        bufs.append((kind, synth.float_terms(40000, kind, seed=3)[None, :]))
    for name, terms in bufs:
        got = np.asarray(run(terms), dtype=np.float32).view(np.uint32)
        for k in range(terms.shape[0]):
            want = sequential_sum_bits(terms[k])
            if int(got[k]) != want:
                fails.append(f"{name}[{k}]: 0x{int(got[k]):08x}, the sequential binary32 sum is 0x{want:08x}")
    return fails


# (terms, expected value) worked by hand from round-to-nearest-even
HAND_WORKED = [
    # 2^24 + 1 lies halfway between 2^24 and 2^24 + 2: the even significand, 2^24
    ([2.0 ** 24, 1.0], 2.0 ** 24),
    ([2.0 ** 24, 1.0, 1.0, 1.0], 2.0 ** 24),
    # 2^24 + 3 lies halfway between 2^24 + 2 (odd significand) and 2^24 + 4
    ([2.0 ** 24, 3.0], 2.0 ** 24 + 4),
    ([2.0 ** 24 + 2, 1.0], 2.0 ** 24 + 4),
    ([2.0 ** 24, 1.5], 2.0 ** 24 + 2),  # above half: up
    # 1 + 2^-24 is halfway between 1 and 1 + 2^-23: stays 1
    ([1.0, 2.0 ** -24], 1.0),
    ([1.0, 2.0 ** -24 + 2.0 ** -47], 1.0 + 2.0 ** -23),
    # the first add rounds up to 1 + 2^-23 (odd), so the second tie goes up
    ([1.0, 2.0 ** -24 + 2.0 ** -47, 2.0 ** -24], 1.0 + 2.0 ** -22),
    # order matters: small terms first add up before the large one
    ([1.0, 2.0 ** 24], 2.0 ** 24),
    ([2.0 ** -24, 2.0 ** -24, 1.0], 1.0 + 2.0 ** -23),
    # subnormals add exactly, into the normal range
    ([2.0 ** -149, 2.0 ** -149], 2.0 ** -148),
    ([2.0 ** -126 - 2.0 ** -149, 2.0 ** -149], 2.0 ** -126),
    # the largest float plus half its last place: a tie with 2^128, whose
    # significand is even, so the sum overflows to infinity
    ([3.4028234663852886e38, 2.0 ** 103], float("inf")),
    ([3.4028234663852886e38, 2.0 ** 102], 3.4028234663852886e38),
    # zeros of either sign change nothing
    ([0.0, -0.0, 0.0], 0.0),
    ([2.5, -0.0, 0.0, 0.5], 3.0),
]


def pin_hand_worked(run):
    """Sums worked by hand around ties, subnormals and overflow."""
    fails = []
    for terms, want in HAND_WORKED:
        t = np.array([terms], dtype=np.float32)
        got = np.asarray(run(t), dtype=np.float32)[0]
        if _bits(got) != _bits(want) or np.signbit(got) != np.signbit(np.float32(want)):
            fails.append(f"{terms}: {got!r}, want {want!r}")
        # the integer emulation agrees with the hand result
        if sequential_sum_bits(t[0]) != _bits(want):
            fails.append(f"{terms}: the emulation disagrees with the hand result")
    return fails


def pin_closed_forms(run):
    """n ones sum to n while n <= 2^24 and then stall at 2^24 (every further
    add is a tie that keeps the even significand); a sum that starts at 2^24
    stays there under terms below 1."""
    fails = []
    for n in (0, 1, 1000, (1 << 24) - 1, 1 << 24, (1 << 24) + 9):
        got = float(np.asarray(run(np.ones((1, n), dtype=np.float32)))[0])
        want = float(min(n, 1 << 24))
        if got != want:
            fails.append(f"{n} ones: {got}, want {want}")
    t = synth.float_terms(100000, "stall", seed=5)[None, :]
    if float(np.asarray(run(t))[0]) != 2.0 ** 24:
        fails.append("the stalled sum moved")
    return fails


def pin_zero_terms_change_nothing(run):
    """Inserting zeros (+0 or -0) anywhere leaves the sum as it was [psnr_hvs
    page, Consequences: adding a zero changes nothing]."""
    fails = []
    rng = np.random.Generator(np.random.PCG64(17))
    base = synth.hvs_like_terms(400, 1, seed=23)[0]
    nz = base[base != 0]
    # the nonzero terms in their order, at sorted random places of a buffer
    # of base's length whose other terms are zeros of random sign; and the
    # nonzero terms first, then plain zeros
    spread = np.where(rng.random(base.size) < 0.5, np.float32(0.0), np.float32(-0.0)).astype(np.float32)
    pos = np.sort(rng.choice(base.size, size=nz.size, replace=False))
    spread[pos] = nz
    nz = np.concatenate([nz, np.zeros(base.size - nz.size, dtype=np.float32)])
    got = np.asarray(run(np.stack([nz, spread, base])), dtype=np.float32)
    if len({_bits(g) for g in got}) != 1:
        fails.append(f"zeros changed the sum: {[hex(_bits(g)) for g in got]}")
    return fails


ALL_PINS = [pin_hand_worked, pin_closed_forms, pin_zero_terms_change_nothing, pin_matches_integer_emulation]


def run_all(run, pins=None):
    """{pin name: failures} for every pin that fails."""
    out = {}
    for pin in pins or ALL_PINS:
        fails = pin(run)
        if fails:
            out[pin.__name__] = fails
    return out
