"""The oracle against what the pages and plain mathematics fix (CPU only)."""
import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)
