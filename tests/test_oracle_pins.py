"""The CPU oracle agrees with everything fixed outside it (runs without a GPU)."""

import pytest

from tests import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()
