"""The CPU oracle against its pins (tests/oracle_pins.py explains each one)."""
import numpy as np
import pytest

from tests import oracle_pins as P


@pytest.fixture
def rng():
    return np.random.default_rng(20261202)


def test_hand_examples(orc):
    P.pin_hand_examples(orc)


def test_metadata_hand(orc):
    P.pin_metadata_hand(orc)


def test_cutoff_boundaries(orc):
    P.pin_cutoff_boundaries(orc)


def test_metadata_closed_forms(orc, rng):
    P.pin_metadata_closed_forms(orc, rng)


def test_mask_zero_is_plain_gather(orc, rng):
    P.pin_mask_zero_is_plain_gather(orc, rng)


def test_full_participation_independent_of_chunk(orc, bmi2, rng):
    P.pin_full_participation_independent_of_chunk(orc, bmi2, rng)


def test_compact(orc, rng):
    P.pin_compact(orc, rng)


def test_compact_aligned(orc, rng):
    P.pin_compact_aligned(orc, rng)


def test_invalid_ids(orc, rng):
    P.pin_invalid_ids(orc, rng)


def test_brute_force(orc, rng):
    P.pin_brute_force(orc, rng)


def test_roundtrip_and_format(orc, bmi2, rng):
    P.pin_roundtrip_and_format(orc, bmi2, rng)


def test_rejects_bad_threshold(orc):
    rows = np.zeros((4, 1), np.uint32)
    for T in (0.49, 1.01, float("nan")):
        with pytest.raises(ValueError):
            orc.build_metadata(rows, T)
