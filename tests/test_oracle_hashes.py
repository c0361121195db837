"""The oracle's results on the workload-shaped seeded inputs against the
recorded SHA-256 baseline (tests/golden/oracle_hashes.json, written by
tests/golden/oracle_hashes.py --record, which runs only the oracle)."""
import pytest

from tests.golden import oracle_hashes as oh


def test_record_covers_every_config():
    rec = oh.load()
    assert set(oh.CONFIGS) <= set(rec)
    for name in oh.CONFIGS:
        assert rec[name], name


@pytest.mark.parametrize("name", oh.CONFIGS)
def test_oracle_matches_recorded_hashes(name):
    rec = oh.load()[name]
    got = oh.compute(name)
    assert sorted(got) == sorted(rec)
    bad = [k for k in rec if got[k] != rec[k]]
    assert not bad, f"{name}: {bad}"
