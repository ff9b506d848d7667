"""The oracle against facts that do not come from the oracle itself."""
import pytest

from oracle import lora as ol
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(ol)


def test_max_rel_err_definition():
    import numpy as np
    assert ol.max_rel_err(np.zeros(3), np.zeros(3)) == 0.0
    assert ol.max_rel_err(np.ones(3), np.zeros(3)) == float("inf")
    assert ol.max_rel_err(np.asarray([1.0, 2.5]), np.asarray([1.0, 2.0])) == 0.25


@pytest.mark.parametrize("pin", __import__("tests.pins_adamw", fromlist=["ALL_PINS"]).ALL_PINS,
                         ids=lambda f: f.__name__)
def test_adamw_pin(pin):
    from oracle import adamw
    pin(adamw)


@pytest.mark.parametrize("pin", __import__("tests.pins_multi", fromlist=["ALL_PINS"]).ALL_PINS,
                         ids=lambda f: f.__name__)
def test_multi_pin(pin):
    from oracle import multi
    pin(multi)


@pytest.mark.parametrize("pin", __import__("tests.pins_mx", fromlist=["ALL_PINS"]).ALL_PINS,
                         ids=lambda f: f.__name__)
def test_mx_pin(pin):
    from oracle import mx
    pin(mx)
