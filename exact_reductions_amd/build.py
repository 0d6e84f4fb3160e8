"""Compile libvqx.so for gfx950 in-tree (hipcc, no JIT cache)."""

from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("plane_stats.hip", "cpu_order.hip", "stage1_mapped.hip", "plane_views.hip", "host_stream.hip",
                                            "float_sum.hip", "vqx_api.hip")]
LIBRARY = os.path.join(HERE, "libvqx.so")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # never fuse a product with an add (the CPU reference is built the same way)
    "-ffp-contract=off",
    "-Wall", "-Wextra", "-Werror", "-Wno-unused-command-line-argument",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def build(verbose: bool = False, save_temps: str | None = None) -> str:
    """Build libvqx.so beside this file and return its path.

    ``save_temps``: a directory that receives the intermediate files,
    including the gfx950 assembly, for inspection.
    """
    tmp = LIBRARY + ".tmp"
    cmd = ["hipcc", *FLAGS, *SOURCES, "-o", tmp]
    cwd = None
    if save_temps:
        os.makedirs(save_temps, exist_ok=True)
        cmd.insert(1, "--save-temps")
        cwd = save_temps
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, cwd=cwd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(line for line in r.stderr.splitlines() if noise not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if verbose and err.strip():
        print(err)
    os.replace(tmp, LIBRARY)
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose=True))
