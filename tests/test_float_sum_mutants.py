"""Planted mistakes in the running float sum must each fail a pin (CPU only).

Each mutant is a plausible wrong way to form the psnr_hvs CPU extractor's
sum: the per-block device sums of the earlier GPU twins, a double
accumulator, numpy's pairwise float sum, a compensated sum (closer to the
exact value, not the CPU's), the terms in reverse order, and a float add that
truncates instead of rounding to nearest even.  The oracle itself passes
every pin (tests/test_float_sum_pins.py).
"""

from __future__ import annotations

import numpy as np
import pytest

import float_sum_pins


def _rows(terms):
    t = np.ascontiguousarray(terms, dtype=np.float32)
    return t if t.ndim == 2 else t[None, :]


def double_accumulator(terms):
    """Sum in double, rounded to float once at the end."""
    return np.array([np.float32(float(np.sum(r.astype(np.float64)))) for r in _rows(terms)], dtype=np.float32)


def pairwise_float(terms):
    """numpy's float32 sum (pairwise blocks)."""
    return np.array([np.sum(r, dtype=np.float32) for r in _rows(terms)], dtype=np.float32)


def block_sums_then_blocks(terms):
    """64-term blocks summed in float, then the block sums added in float."""
    out = []
    for r in _rows(terms):
        pad = np.zeros(-(-r.size // 64) * 64, dtype=np.float32)
        pad[:r.size] = r
        blocks = np.cumsum(pad.reshape(-1, 64), axis=1, dtype=np.float32)[:, -1] if pad.size else pad
        out.append(np.cumsum(blocks, dtype=np.float32)[-1] if blocks.size else np.float32(0))
    return np.array(out, dtype=np.float32)


def compensated(terms):
    """Kahan's compensated float sum."""
    out = []
    for r in _rows(terms):
        s = np.float32(0)
        c = np.float32(0)
        with np.errstate(over="ignore", invalid="ignore"):
            for t in r.tolist():
                y = np.float32(np.float32(t) - c)
                u = np.float32(s + y)
                c = np.float32(np.float32(u - s) - y)
                s = u
        out.append(s)
    return np.array(out, dtype=np.float32)


def reverse_order(terms):
    """The right running sum, over the terms in reverse order."""
    return np.array([np.cumsum(r[::-1], dtype=np.float32)[-1] if r.size else np.float32(0)
                     for r in _rows(terms)], dtype=np.float32)


def truncating_add(terms):
    """A running sum whose adds truncate (round toward zero) instead of
    rounding to nearest even, in the integer form of the pins' emulation."""
    out = []
    for r in _rows(terms):
        s = 0
        for b in r.view(np.uint32).tolist():
            if s == float_sum_pins.INF_BITS or b == float_sum_pins.INF_BITS:
                s = float_sum_pins.INF_BITS
                continue
            b = 0 if b == 0x80000000 else b
            x = float_sum_pins._units(s) + float_sum_pins._units(b)
            k = x.bit_length() - 24
            if k > 0:
                x = (x >> k) << k
            s = float_sum_pins._round_to_binary32(x)
        out.append(np.uint32(s).view(np.float32))
    return np.array(out, dtype=np.float32)


def running_sum(terms):
    """The unmutated definition in numpy: cumsum adds in order, in float32."""
    return np.array([np.cumsum(r, dtype=np.float32)[-1] if r.size else np.float32(0)
                     for r in _rows(terms)], dtype=np.float32)


MUTANTS = [double_accumulator, pairwise_float, block_sums_then_blocks, compensated, reverse_order,
           truncating_add]


def test_unmutated_numpy_running_sum_passes_every_pin():
    with np.errstate(over="ignore"):
        assert float_sum_pins.run_all(running_sum) == {}


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_mutant_fails_a_pin(mutant):
    with np.errstate(over="ignore"):
        # the slow (pure-Python) mutants skip the pin over long buffers
        pins = [p for p in float_sum_pins.ALL_PINS
                if not (mutant in (compensated, truncating_add) and p is float_sum_pins.pin_closed_forms)]
        fails = {}
        for pin in pins:
            f = pin(mutant)
            if f:
                fails[pin.__name__] = f
                break
    assert fails, f"{mutant.__name__} passes every pin"
