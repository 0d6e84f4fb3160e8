"""Write oracle_sums.json: the oracle's outputs on small seeded inputs.

Calls only ``oracle`` (and ``synth`` for the inputs).  The stored values pin
the oracle against later edits of its own arithmetic; every input is named
by its recipe and sha256.  Run from the repository root:

    python tests/golden/make_golden.py
"""

from __future__ import annotations

import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402


def cases():
    yield "workload1_full", 8, synth.generate(1)
    for n in (2, 3, 4, 5):
        wl = synth.WORKLOADS[n]
        yield f"workload{n}_2x96x64", wl.bpc, synth.generate(n, nframes=2, w=96, h=64)
    yield "ties_4097", 16, synth.constant_pair(7, 3, 1, 16, 4097, 0)
    yield "worst_65535_vs_0", 16, synth.constant_pair(5, 5, 1, 16, 65535, 0)
    yield "bpc13_container_max_31x17", 13, synth.uniform_planes(31, 17, 2, 13, seed=1313, container_max=True)


def main():
    out = []
    for name, bpc, (ref, dist) in cases():
        seq = oracle.seq_batch_sums(ref, dist, bpc)
        ex = oracle.exact_batch_sums(ref, dist)
        out.append({
            "name": name, "bpc": bpc, "shape": list(ref.shape), "sha256": synth.sha256(ref, dist),
            "exact": [[str(int(v)) for v in row] for row in ex],
            "seq_hex": [[float(v).hex() for v in row] for row in seq],
        })
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_sums.json")
    with open(path, "w") as f:
        json.dump({"_about": "written by tests/golden/make_golden.py from oracle/ only", "cases": out}, f, indent=1)
    print(path)


if __name__ == "__main__":
    main()
