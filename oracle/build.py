"""Compile the C oracle (test infrastructure only).

gcc -O2 with contraction off and no fast-math: the CPU extractors the oracle
stands for are built that way ("ADR-1397: GPU psnr_hvs twins reproduce the
CPU's running float sum bit for bit", Decision).
"""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
SOURCES = [os.path.join(HERE, f) for f in ("float_sums.c", "running_float_sum.c")]
LIBRARY = os.path.join(HERE, "libfloat_sums.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fno-unsafe-math-optimizations",
          "-Wall", "-Wextra", "-Werror", "-shared", "-fPIC"]


def build(verbose: bool = False) -> str:
    """Compile the C sources into libfloat_sums.so beside them; return its path."""
    tmp = LIBRARY + ".tmp"
    cmd = ["gcc", *CFLAGS, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
