"""Seeded random sweeps of the entry points against the oracle (marked gpu).

Each seed draws a few dozen batches of random depth, size (1 sample wide
to a few thousand), frame count and content (the whole container, bright,
dark, constant, a dark tenth among bright samples) and checks:
  * the exact sums of the contiguous entry point against O2, integer for
    integer;
  * every few batches (depths 9..16), the CPU-order form: its exact sums
    against O2 and its CPU sums against O1's sequential doubles, bit for bit;
  * views with random pitches, offsets and frame strides (0 too): the five
    sums against O2 and the integer psnr twin against O3.
The draws are seeded, so every run checks the same batches.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

from exact_reductions_amd import vqx  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    vqx.lib()  # raises if libvqx.so is missing: no fallback exists


KINDS = ("uniform", "container", "bright", "dark", "const", "mixed")


def _content(rng, shape, bpc, kind):
    hi = (1 << bpc) - 1
    if kind == "uniform":
        return rng.integers(0, hi, size=shape, endpoint=True)
    if kind == "container":
        return rng.integers(0, 255 if bpc == 8 else 65535, size=shape, endpoint=True)
    if kind == "bright":
        return rng.integers(hi - hi // 5, hi, size=shape, endpoint=True)
    if kind == "dark":
        return rng.integers(0, max(1, hi // 20), size=shape, endpoint=True)
    if kind == "const":
        return np.full(shape, int(rng.integers(0, hi + 1)))
    dark = rng.random(shape) < 0.1
    return np.where(dark, rng.integers(0, max(1, hi // 16), size=shape, endpoint=True),
                    rng.integers(hi // 2, hi, size=shape, endpoint=True))


def _dev(a):
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).cuda()


def _o2_rows(ref, dist):
    return oracle.exact_batch_sums(np.ascontiguousarray(ref), np.ascontiguousarray(dist))


@pytest.mark.parametrize("seed", range(8))
def test_random_contiguous_batches(seed):
    rng = np.random.default_rng(90_000 + seed)
    for case in range(24):
        bpc = int(rng.integers(8, 17))
        dt = np.uint8 if bpc == 8 else np.uint16
        w = int(rng.choice([rng.integers(1, 64), rng.integers(64, 1500), rng.integers(1500, 4100)]))
        h = int(rng.integers(1, max(2, min(2000, 1_500_000 // w))))
        f = int(rng.integers(1, 5))
        kr, kd = rng.choice(KINDS), rng.choice(KINDS)
        ref = _content(rng, (f, h, w), bpc, kr).astype(dt)
        dist = _content(rng, (f, h, w), bpc, kd).astype(dt)
        label = f"seed {seed} case {case}: bpc {bpc} {w}x{h}x{f} {kr}/{kd}"
        R, D = _dev(ref), _dev(dist)
        noise, moments = vqx.plane_stats_batch(R, D, bpc)
        torch.cuda.synchronize()
        o2 = _o2_rows(ref, dist)
        got = np.concatenate([noise.cpu().numpy()[:, None], moments.cpu().numpy()], axis=1)
        assert np.array_equal(got, o2), label
        if bpc > 8 and case % 3 == 0:
            n, m, cn, cm = vqx.plane_stats_batch_cpu_order(R, D, bpc)
            torch.cuda.synchronize()
            assert np.array_equal(np.concatenate([n.cpu().numpy()[:, None], m.cpu().numpy()], axis=1), o2), label
            o1 = oracle.seq_batch_sums(ref, dist, bpc)
            s = 1 << (bpc - 8)
            cpu = np.concatenate([cn.cpu().numpy()[:, None], cm.cpu().numpy()], axis=1)
            for i in range(f):
                for k, p in enumerate(oracle.UNIT_POWER):
                    want = float(o1[i][k]) * float(s ** p)
                    assert float(cpu[i][k]) == want and int(cpu[i][k]) == int(want), f"{label} frame {i} output {k}"


@pytest.mark.parametrize("seed", range(8))
def test_random_views(seed):
    rng = np.random.default_rng(91_000 + seed)
    for case in range(60):
        bpc = int(rng.integers(8, 17))
        dt = np.uint8 if bpc == 8 else np.uint16
        w, h, f = int(rng.integers(1, 1500)), int(rng.integers(1, 300)), int(rng.integers(1, 5))
        pr, pd = w + int(rng.integers(0, 40)), w + int(rng.integers(0, 40))
        xr, xd, y0 = int(rng.integers(0, 24)), int(rng.integers(0, 24)), int(rng.integers(0, 3))
        same = bool(rng.random() < 0.2)
        fb = 1 if same else f
        hi = (1 << bpc) - 1
        big_r = rng.integers(0, hi, size=(fb, h + y0, pr + xr), endpoint=True).astype(dt)
        big_d = rng.integers(0, hi, size=(fb, h + y0, pd + xd), endpoint=True).astype(dt)
        R = _dev(big_r)[:, y0:y0 + h, xr:xr + w]
        D = _dev(big_d)[:, y0:y0 + h, xd:xd + w]
        rn, dn = big_r[:, y0:y0 + h, xr:xr + w], big_d[:, y0:y0 + h, xd:xd + w]
        if same:
            R, D = R.expand(f, h, w), D.expand(f, h, w)
            rn, dn = np.broadcast_to(rn, (f, h, w)), np.broadcast_to(dn, (f, h, w))
        label = f"seed {seed} case {case}: bpc {bpc} {w}x{h}x{f} pitches {pr},{pd} at {xr},{xd},{y0} same {same}"
        noise, moments = vqx.plane_stats_view(R, D, bpc)
        inoise = vqx.psnr_int_view(R, D, bpc)
        torch.cuda.synchronize()
        got = np.concatenate([noise.cpu().numpy()[:, None], moments.cpu().numpy()], axis=1)
        assert np.array_equal(got, _o2_rows(rn, dn)), label
        want = np.array([oracle.int_noise(rn[i], dn[i]) for i in range(f)], dtype=np.int64)
        assert np.array_equal(inoise.cpu().numpy(), want), label
