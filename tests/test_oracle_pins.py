"""The fp64 oracle against what the pages and the mathematics fix (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    check()
