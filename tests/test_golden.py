"""The oracle against its recorded outputs on the single-linear workload (CPU).

The fixture is not a pin (the pages print no worked example of the merge); it guards
against unintended changes to the oracle's arithmetic.  A deliberate change
regenerates it with tests/golden/make_golden.py.
"""
import os

from tests.golden.make_golden import FIXTURE, compute


def test_oracle_matches_recorded_fixture():
    rec = {}
    with open(FIXTURE) as fh:
        for line in fh:
            if line.startswith("#") or "=" not in line:
                continue
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    assert rec == compute()
