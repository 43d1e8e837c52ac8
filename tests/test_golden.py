"""The oracle still reproduces its stored tiny-workload outputs (regression guard)."""
import json
import os

from tests.golden.make_golden import compute


def test_tiny_oracle_unchanged():
    path = os.path.join(os.path.dirname(__file__), "golden", "tiny_oracle.json")
    with open(path) as f:
        stored = json.load(f)
    assert compute() == stored
