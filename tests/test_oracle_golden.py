"""The oracle reproduces its stored outputs (tests/golden/oracle_sums.json)."""

import json
import os

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def _cases():
    import make_golden  # noqa: F401  (tests/golden is put on sys.path below)
    return {name: (bpc, planes) for name, bpc, planes in make_golden.cases()}


def _stored():
    with open(os.path.join(HERE, "golden", "oracle_sums.json")) as f:
        return json.load(f)["cases"]


@pytest.fixture(scope="module")
def inputs():
    import sys
    sys.path.insert(0, os.path.join(HERE, "golden"))
    return _cases()


@pytest.mark.parametrize("case", _stored(), ids=lambda c: c["name"])
def test_oracle_matches_stored(case, inputs):
    import synth
    bpc, (ref, dist) = inputs[case["name"]]
    assert synth.sha256(ref, dist) == case["sha256"], "the generator changed"
    ex = oracle.exact_batch_sums(ref, dist)
    seq = oracle.seq_batch_sums(ref, dist, bpc)
    assert [[str(int(v)) for v in row] for row in ex] == case["exact"]
    assert [[float(v).hex() for v in row] for row in seq] == case["seq_hex"]
