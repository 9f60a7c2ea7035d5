"""The CPU oracle against the facts the design spec and mathematics fix
(closed forms, textbook rounding, hand-derived detectors, invariants,
brute force).  CPU only."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()
