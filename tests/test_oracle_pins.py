"""The oracle against its pins (CPU only)."""
import pytest

import oracle
import oracle_pins as P


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("check", [c for c in P.ALL_CHECKS], ids=lambda c: c.__name__)
def test_pin(lib, check):
    check(lib)


def test_products_exact():
    P.check_products_exact()
