"""The step-by-step models of the pages' kernels against the pages' own facts
(the pins in tests/model_pins.py, run on oracle/models.py: every one must
hold)."""

import pytest

from oracle import models

import model_pins


@pytest.mark.parametrize("pin", model_pins.PINS, ids=lambda p: p.__name__)
def test_model_pin_holds(pin):
    pin(models)
