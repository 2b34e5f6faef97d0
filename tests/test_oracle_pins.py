"""The fp64 oracle against results fixed by the pages and by mathematics (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("check", pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check()
