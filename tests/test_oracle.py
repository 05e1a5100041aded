"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    ok, detail = pin(oracle.cca_oracle)
    assert ok, detail


import oracle.cca_serving
from tests import serving_pins


@pytest.mark.parametrize("pin", serving_pins.ALL_SERVING_PINS, ids=lambda f: f.__name__)
def test_serving_pin(pin):
    ok, detail = pin(oracle.cca_serving)
    assert ok, detail


import oracle.cca_backward
from tests import backward_pins


@pytest.mark.parametrize("pin", backward_pins.ALL_BACKWARD_PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    ok, detail = pin(oracle.cca_backward)
    assert ok, detail


import oracle.cca_lca
from tests import lca_pins


@pytest.mark.parametrize("pin", lca_pins.ALL_LCA_PINS, ids=lambda f: f.__name__)
def test_lca_pin(pin):
    ok, detail = pin(oracle.cca_lca)
    assert ok, detail
