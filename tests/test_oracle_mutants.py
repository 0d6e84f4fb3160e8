"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

The mutants are variants of a numpy re-expression of the oracle's
arithmetic (binary32 terms, a sequential float64 running sum via cumsum),
each with one plausible mistake: the defects the pages report in earlier GPU
twins (fp32 block sums, exact integer squares, stale accumulators), and the
generic ones (a dropped term, a wrong sign, a transposed operand, a wrong
scale, a wrong rounding, a double sum in another order).  The unmutated
re-expression must pass every pin.  A double sum in another order changes
nothing below 2^53 and stays within the bound past it, so only the pin of
the CPU's raster order past 2^53 may catch it.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle_pins

F32 = np.float32


class NumpyOracle:
    """The oracle's arithmetic in vectorized numpy; mutants override pieces."""

    def scaler(self, bpc):
        return F32(1 << (bpc - 8))

    def samples(self, plane, bpc):
        return plane.astype(F32) / self.scaler(bpc)

    def diff(self, r, d):
        return r - d

    def square(self, x):
        return x * x

    def terms(self, ref, dist, bpc):
        r = self.samples(ref, bpc)
        d = self.samples(dist, bpc)
        e = self.diff(r, d)
        return [self.square(e), r, d, self.square(r), self.square(d)]

    def reduce(self, t, k):
        return float(np.cumsum(t.astype(np.float64).ravel())[-1]) if t.size else 0.0

    def frame(self, ref, dist, bpc):
        return [self.reduce(t, k) for k, t in enumerate(self.terms(ref, dist, bpc))]

    def seq(self, ref, dist, bpc):
        return np.array([self.frame(ref[f], dist[f], bpc) for f in range(ref.shape[0])])

    def exact(self, ref, dist):
        return oracle.exact_batch_sums(ref, dist)

    def q(self, n):
        return oracle.q_int(n)

    def bound(self, pixels, e, bpc):
        return oracle.past53_bound(pixels, e, bpc)


def _blocks(t, b):
    h, w = t.shape
    hp, wp = -(-h // b) * b, -(-w // b) * b
    p = np.zeros((hp, wp), dtype=t.dtype)
    p[:h, :w] = t
    return p.reshape(hp // b, b, wp // b, b).transpose(0, 2, 1, 3).reshape(-1, b * b)


class M1Fp32BlockSums(NumpyOracle):
    """The old float_psnr twin: fp32 sums per 16x16 block, blocks in double."""

    def reduce(self, t, k):
        blocks = np.cumsum(_blocks(t, 16), axis=1, dtype=F32)[:, -1]
        return float(np.cumsum(blocks.astype(np.float64))[-1])


class M2ExactIntegerSquares(NumpyOracle):
    """The old float_moment twin: exact squares (no rounding to 24 bits)."""

    def terms(self, ref, dist, bpc):
        t = super().terms(ref, dist, bpc)
        s2 = float(self.scaler(bpc)) ** 2
        t[3] = ref.astype(np.float64) ** 2 / s2
        t[4] = dist.astype(np.float64) ** 2 / s2
        return t


class M3U32BlockWrap(NumpyOracle):
    """One uint32 per 256-term block at every depth: block sums wrap mod 2^32."""

    def reduce(self, t, k):
        if k not in (0, 3, 4):
            return super().reduce(t, k)
        s2 = 2.0 ** (2 * self.bpc_now - 16)
        units = (t.astype(np.float64) * s2).astype(np.int64)
        blocks = _blocks(units, 16).sum(axis=1) % (1 << 32)
        return float(int(blocks.sum())) / s2

    def frame(self, ref, dist, bpc):
        self.bpc_now = bpc
        return super().frame(ref, dist, bpc)


def _round24(n, mode):
    n = int(n)
    if n < (1 << 24):
        return n
    k = n.bit_length() - 24
    q, r = divmod(n, 1 << k)
    if mode == "truncate":
        pass
    elif mode == "ties_away":
        if r >= (1 << (k - 1)):
            q += 1
    return q << k


class M4TruncatedSquare(NumpyOracle):
    """Float square rounded toward zero instead of to nearest even."""

    def square(self, x):
        return self._rounded(x, "truncate")

    def _rounded(self, x, mode):
        # x holds multiples of 1/scaler; work in integer units of the sample
        scale = self.unit
        n = np.rint(np.abs(x.astype(np.float64)) * scale).astype(np.int64)
        sq = np.vectorize(lambda v: _round24(v * v, mode), otypes=[np.int64])(n)
        return (sq.astype(np.float64) / (scale * scale)).astype(F32)

    def terms(self, ref, dist, bpc):
        self.unit = float(1 << (bpc - 8))
        return super().terms(ref, dist, bpc)


class M4bTiesAwaySquare(M4TruncatedSquare):
    """Float square rounded half away from zero instead of half to even."""

    def square(self, x):
        return self._rounded(x, "ties_away")


class M5PairwiseDouble(NumpyOracle):
    """A double sum in another (pairwise) order."""

    def reduce(self, t, k):
        return float(np.sum(t.astype(np.float64)))


class M5bColumnMajor(NumpyOracle):
    """One running double, visiting the plane column by column."""

    def reduce(self, t, k):
        return float(np.cumsum(t.astype(np.float64).T.ravel())[-1]) if t.size else 0.0


class M5cRowPartials(NumpyOracle):
    """Each row summed into its own double, the row sums then added in order."""

    def reduce(self, t, k):
        rows = np.cumsum(t.astype(np.float64), axis=1)[:, -1]
        return float(np.cumsum(rows)[-1]) if t.size else 0.0


class M6NoResetBetweenFrames(NumpyOracle):
    """Accumulators carried from one frame into the next (no clear)."""

    def seq(self, ref, dist, bpc):
        out, carry = [], np.zeros(5)
        for f in range(ref.shape[0]):
            carry = carry + np.array(self.frame(ref[f], dist[f], bpc))
            out.append(carry.copy())
        return np.array(out)


class M7DropLastColumn(NumpyOracle):
    """The last column of every row is skipped."""

    def terms(self, ref, dist, bpc):
        return super().terms(ref[:, :-1], dist[:, :-1], bpc)


class M8WrongSign(NumpyOracle):
    """The difference is taken as a sum."""

    def diff(self, r, d):
        return r + d


class M9SwappedMoments(NumpyOracle):
    """The reference moments are taken from the distorted plane."""

    def terms(self, ref, dist, bpc):
        t = super().terms(ref, dist, bpc)
        return [t[0], t[2], t[1], t[4], t[3]]


class M10UnscaledSamples(NumpyOracle):
    """Samples are not divided by the scaler."""

    def samples(self, plane, bpc):
        return plane.astype(F32)


class M11ScaledOnce(NumpyOracle):
    """Squares divided by the scaler once instead of twice."""

    def square(self, x):
        return (x * x) * self.s_now

    def terms(self, ref, dist, bpc):
        self.s_now = self.scaler(bpc)
        return super().terms(ref, dist, bpc)


class M12NoiseInDouble(NumpyOracle):
    """Squared difference taken in double (no rounding to 24 bits)."""

    def terms(self, ref, dist, bpc):
        t = super().terms(ref, dist, bpc)
        s = float(self.scaler(bpc))
        e = (ref.astype(np.float64) - dist.astype(np.float64)) / s
        t[0] = e * e
        return t


class M13WrappedDifference(NumpyOracle):
    """Difference taken in the sample's unsigned type (wraps around)."""

    def terms(self, ref, dist, bpc):
        t = super().terms(ref, dist, bpc)
        wrapped = (ref - dist).astype(F32) / self.scaler(bpc)
        t[0] = wrapped * wrapped
        return t


class X1QTiesAway(NumpyOracle):
    """The integer oracle rounds squares half away from zero."""

    def q(self, n):
        return _round24(n * n, "ties_away")


class X2QTruncate(NumpyOracle):
    """The integer oracle truncates squares to 24 bits."""

    def q(self, n):
        return _round24(n * n, "truncate")


class X3ExactOffByOne(NumpyOracle):
    """The integer oracle looks the square up one entry too far."""

    def exact(self, ref, dist):
        t = oracle.q_table()
        out = []
        for f in range(ref.shape[0]):
            r = ref[f].astype(np.int64).ravel()
            d = dist[f].astype(np.int64).ravel()
            idx = np.minimum(np.abs(r - d) + 1, 65535)
            out.append([int(t[idx].sum()), int(r.sum()), int(d.sum()), int(t[r].sum()), int(t[d].sum())])
        return np.array(out, dtype=np.int64)


class X4ExactMomentsSwapped(NumpyOracle):
    """The integer oracle returns the dist square sum as the ref's."""

    def exact(self, ref, dist):
        e = oracle.exact_batch_sums(ref, dist)
        return e[:, [0, 1, 2, 4, 3]]


class B1BoundWithoutUnit(NumpyOracle):
    """Bound that forgets the 2^-16 unit of a 16-bit second moment."""

    def bound(self, pixels, e, bpc):
        return (pixels - (1 << 21) + 1) / pixels * 2.0 ** (e - 53) + 2.0 ** -37


class B2BoundWithoutExactPrefix(NumpyOracle):
    """Bound that counts every add as rounding (drops the exact first 2^21)."""

    def bound(self, pixels, e, bpc):
        return 2.0 ** (e - 69) + 2.0 ** -37


MUTANTS = [M1Fp32BlockSums, M2ExactIntegerSquares, M3U32BlockWrap, M4TruncatedSquare,
           M4bTiesAwaySquare, M6NoResetBetweenFrames, M7DropLastColumn, M8WrongSign,
           M9SwappedMoments, M10UnscaledSamples, M11ScaledOnce, M12NoiseInDouble,
           M13WrappedDifference, X1QTiesAway, X2QTruncate, X3ExactOffByOne,
           X4ExactMomentsSwapped, B1BoundWithoutUnit, B2BoundWithoutExactPrefix,
           M5PairwiseDouble, M5bColumnMajor, M5cRowPartials]

# The cheap pins first; a mutant stops at its first failing pin.
FAST_FIRST = sorted(oracle_pins.ALL_PINS, key=lambda p: p in oracle_pins.SLOW_PINS)


def _first_failure(impl):
    for pin in FAST_FIRST:
        if isinstance(impl, (M4TruncatedSquare,)) and pin in oracle_pins.SLOW_PINS:
            continue  # per-sample Python rounding is too slow at 4K; other pins catch it
        fails = pin(impl)
        if fails:
            return pin.__name__, fails
    return None


def test_unmutated_reexpression_passes_every_pin():
    assert oracle_pins.run_all(NumpyOracle()) == {}


@pytest.mark.parametrize("order", [M5PairwiseDouble, M5bColumnMajor, M5cRowPartials],
                         ids=["pairwise", "column_major", "row_partials"])
def test_other_summation_order_fails_only_the_raster_order_pin(order):
    """A double sum in another order equals the sequential one below 2^53 and
    stays within the bound past it; only the CPU's own order of roundings past
    2^53 [float_psnr page, Consequences] tells it apart."""
    fails = oracle_pins.run_all(order())
    assert set(fails) == {"pin_past53_raster_order", "pin_past53_bound_below_16_bits"}, fails
    # within the bound at every depth: only the bit-for-bit order checks fail
    assert all("emulation" in f for f in fails["pin_past53_bound_below_16_bits"]), fails


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_mutant_fails_a_pin(mutant):
    assert _first_failure(mutant()) is not None, f"{mutant.__name__} passes every pin"


def test_m1_passes_at_8_bits_and_fails_at_10():
    """The fp32-block defect is invisible on 8-bit noise and visible on
    full-range 10-bit noise [float_psnr page, Context and Consequences]."""
    import synth
    m1 = M1Fp32BlockSums()
    for bpc, want_equal in ((8, True), (10, False)):
        ref, dist = synth.uniform_planes(64, 64, 1, bpc, seed=9 + bpc)
        exact = oracle.exact_batch_sums(ref, dist)[0]
        scale = float((1 << (bpc - 8)) ** 2)
        equal = m1.seq(ref, dist, bpc)[0, 0] == float(int(exact[0])) / scale
        assert equal == want_equal, f"bpc {bpc}"


def test_m2_passes_up_to_12_bits_and_fails_at_16():
    """Exact integer squares equal the float squares up to 12 bits, not at 16
    [float_moment page, Context]."""
    import synth
    m2 = M2ExactIntegerSquares()
    for bpc, want_equal in ((12, True), (16, False)):
        ref, dist = synth.uniform_planes(64, 64, 1, bpc, seed=19 + bpc)
        exact = oracle.exact_batch_sums(ref, dist)[0]
        scale = float((1 << (bpc - 8)) ** 2)
        equal = m2.seq(ref, dist, bpc)[0, 3] == float(int(exact[3])) / scale
        assert equal == want_equal, f"bpc {bpc}"
