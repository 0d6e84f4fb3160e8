"""TEST INFRASTRUCTURE ONLY: oracle of the integer psnr twin.

Only the tests, the smoke check and the bench's cpu_baseline leg may use this
module; no product code path does.  It shares no code with the HIP library.

Sources (web pages, cited by title and section):

* [PSNR] "ADR-1440: float_psnr_hip adds its squared differences as integers
  and returns the CPU's score bit for bit" -- Alternatives (the integer
  psnr twin keeps one uint64 per frame), Context (scaler, the 8-bit scale of
  float_psnr), Consequences (the capped and uncapped scores).

What is computed here (readings; the pages give no code for integer psnr):

* The noise of a plane is the sum over its samples of (ref - dist)^2, each
  square an exact integer, in one integer per frame.  Samples are the stored
  integers; nothing is scaled, and no square rounds (a difference of two
  16-bit samples squares to less than 2^32, and 2^25 of them sum to less
  than 2^57).  It equals float_psnr's noise in units of 1/scaler^2 wherever
  the float square is exact, i.e. wherever |ref - dist| < 4096.
* The score: mse = noise / (w*h) in double (the integer converted once,
  rounding to nearest even, then one division); psnr = 10*log10(peak^2/mse)
  with peak = 2^bpc - 1 on the stored scale, capped at psnr_max when
  psnr_max > 0; mse = 0 gives psnr_max, or +inf uncapped.  The ratio
  peak^2/mse is float_psnr's, taken on the stored scale instead of the 8-bit
  one.
* A plane is any 2-D array: chroma planes, a region of interest or a plane
  read with a row pitch are the same function of the selected samples.
"""

from __future__ import annotations

import math

import numpy as np


def int_noise(ref: np.ndarray, dist: np.ndarray) -> int:
    """Exact sum of (ref - dist)^2 over one plane, as a Python int."""
    r = np.asarray(ref).astype(np.int64)
    d = np.asarray(dist).astype(np.int64)
    if r.shape != d.shape:
        raise ValueError("ref and dist differ in shape")
    if r.size and (r.min() < 0 or r.max() > 65535 or d.min() < 0 or d.max() > 65535):
        raise ValueError("samples must be 0..65535")
    e = (r - d).ravel()
    return int((e * e).sum())  # int64 is exact: every partial sum stays below 2^57


def int_noise_batch(ref: np.ndarray, dist: np.ndarray) -> np.ndarray:
    """[nframes] int64 noise of a ``[nframes][h][w]`` batch of planes."""
    return np.array([int_noise(ref[f], dist[f]) for f in range(ref.shape[0])], dtype=np.int64)


def int_mse(noise: int, w: int, h: int) -> float:
    """noise / (w*h) in double: one rounding of the integer, one division."""
    return float(int(noise)) / float(w * h)


def int_psnr_db(noise: int, w: int, h: int, bpc: int, psnr_max: float = 0.0) -> float:
    """10*log10(peak^2/mse), peak = 2^bpc - 1, capped at psnr_max > 0."""
    if not 8 <= bpc <= 16:
        raise ValueError("bpc must be 8..16")
    mse = int_mse(noise, w, h)
    if mse == 0.0:
        return psnr_max if psnr_max > 0 else math.inf
    p = float((1 << bpc) - 1)
    v = 10.0 * math.log10(p * p / mse)
    return min(v, psnr_max) if psnr_max > 0 else v
