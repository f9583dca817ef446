"""The CPU oracle against its pins (closed forms, invariants, finite
differences, torch binary64, exact rational rounding).  CPU only."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(orc, check):
    check(orc)


def test_oracle_is_binary64_and_plain(orc):
    # the library exists and reports its OpenMP thread count (used only for
    # the CPU baseline's "cores" figure)
    assert orc.num_threads() >= 1
