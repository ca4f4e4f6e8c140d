"""The oracle's outputs on small seeded workloads match the stored digests
(written by tests/golden/make_oracle_digests.py from the oracle alone)."""
import json
import os

from tests.golden import make_oracle_digests as G


def test_oracle_digests_unchanged():
    with open(G.OUT) as f:
        stored = json.load(f)
    assert G.digests() == stored
