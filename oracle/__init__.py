"""TEST INFRASTRUCTURE ONLY: the CPU oracle for the bit-exact plane reductions.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product (``exact_reductions_amd``)
never does, and this package imports nothing from it.

Two independent forms of the same definition:

* ``seq_*`` -- O1, the CPU's own arithmetic: float samples divided by the
  scaler, float squares, one running double per output in raster order
  (``float_sums.c``).
* ``exact_*`` -- O2, the exact integer sums with an integer-only
  round-to-24-bits for the float square (``exact.py``).
* ``int_*`` -- O3, the integer psnr twin: exact sums of (ref - dist)^2 and
  their score (``int_psnr.py``).
* ``running_float_sums`` -- O4, the running binary32 sum of a buffer of
  float terms, added one by one in buffer order (``running_float_sum.c``),
  as the psnr_hvs CPU extractor sums its terms.

Below 2^53 units the two agree bit for bit; past it O1 is the CPU's rounded
value and O2 the exact one, within ``past53_bound``.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build
from .exact import (  # noqa: F401
    NOISE, REF_SUM, DIST_SUM, REF_SQ, DIST_SQ, TWO53, UNIT_POWER,
    acceptance, binade, conclude_from_doubles, conclude_from_ints, exact_batch_sums,
    exact_frame_sums, past53_bound, peak, psnr_db, q_int, q_table, rne24, scaler,
)
from .int_psnr import int_mse, int_noise, int_noise_batch, int_psnr_db  # noqa: F401

_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIBRARY):
            _build.build()
        lib = ctypes.CDLL(_build.LIBRARY)
        for name in ("oracle_frame_sums",):
            fn = getattr(lib, name)
            fn.restype = ctypes.c_int
            fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                           ctypes.c_int, ctypes.c_void_p]
        lib.oracle_running_float_sums.restype = ctypes.c_int
        lib.oracle_running_float_sums.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int,
                                                  ctypes.c_void_p]
        lib.oracle_batch_sums.restype = ctypes.c_int
        lib.oracle_batch_sums.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_void_p]
        _lib = lib
    return _lib


def _check_planes(ref, dist, bpc):
    dtype = np.uint8 if bpc == 8 else np.uint16
    ref = np.ascontiguousarray(ref)
    dist = np.ascontiguousarray(dist)
    if ref.dtype != dtype or dist.dtype != dtype:
        raise TypeError(f"bpc {bpc} wants {np.dtype(dtype).name} samples")
    if ref.shape != dist.shape:
        raise ValueError("ref and dist differ in shape")
    return ref, dist


def seq_frame_sums(ref: np.ndarray, dist: np.ndarray, bpc: int) -> np.ndarray:
    """O1 for one ``[h][w]`` frame: the five CPU doubles on the 8-bit scale."""
    ref, dist = _check_planes(ref, dist, bpc)
    h, w = ref.shape
    out = np.zeros(5, dtype=np.float64)
    rc = _load().oracle_frame_sums(ref.ctypes.data, dist.ctypes.data, w, h, bpc, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_frame_sums rejected its arguments")
    return out


def seq_batch_sums(ref: np.ndarray, dist: np.ndarray, bpc: int) -> np.ndarray:
    """O1 for a ``[nframes][h][w]`` batch: ``[nframes][5]`` doubles."""
    ref, dist = _check_planes(ref, dist, bpc)
    f, h, w = ref.shape
    out = np.zeros((f, 5), dtype=np.float64)
    rc = _load().oracle_batch_sums(ref.ctypes.data, dist.ctypes.data, w, h, bpc, f, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_batch_sums rejected its arguments")
    return out


def running_float_sums(terms: np.ndarray) -> np.ndarray:
    """O4: for ``[nsums][n]`` float32 terms, the ``[nsums]`` float32 values of
    a binary32 accumulator after each buffer's terms are added one by one,
    in order, from zero."""
    terms = np.ascontiguousarray(terms, dtype=np.float32)
    if terms.ndim == 1:
        terms = terms[None, :]
    nsums, n = terms.shape
    out = np.zeros(nsums, dtype=np.float32)
    rc = _load().oracle_running_float_sums(terms.ctypes.data, n, nsums, out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_running_float_sums rejected its arguments")
    return out
