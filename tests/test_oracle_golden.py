"""The oracle against its stored results (tests/golden/oracle_regression.json,
written by tests/golden/make_golden.py from oracle/ only): a change to the
oracle's arithmetic, or to the seeded generators, fails here."""
import json
import os

from tests.golden import make_golden


def test_oracle_matches_stored_results():
    with open(make_golden.OUT) as f:
        stored = json.load(f)
    now = make_golden.build()
    assert len(now["cases"]) == len(stored["cases"])
    for a, b in zip(now["cases"], stored["cases"]):
        assert a == b, (b["workload"], b["threshold"])


def test_fixture_is_small():
    assert os.path.getsize(make_golden.OUT) < 16384
