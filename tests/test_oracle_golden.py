"""Regression pin: the oracle's outputs on the seeded tiny workload match the
digests that tests/golden/make_golden.py wrote (it calls only the oracle)."""
import json
import os

from tests.golden.make_golden import run

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_matches_golden_digests():
    with open(os.path.join(HERE, "golden", "oracle_tiny.json")) as f:
        ref = json.load(f)
    assert run() == ref
