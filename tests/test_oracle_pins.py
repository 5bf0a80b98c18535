"""The oracle against brute force, closed forms, torch's CPU attention, the
definition's invariants and the values the pages print."""

import pytest

import oracle
from oracle import rules
import _pins


@pytest.mark.parametrize("pin", _pins.ATTENTION_PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("pin", _pins.RULE_PINS, ids=lambda f: f.__name__)
def test_rule_pin(pin):
    pin(rules)


@pytest.mark.parametrize("pin", _pins.CACHE_PINS, ids=lambda f: f.__name__)
def test_cache_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("pin", _pins.VARLEN_PINS, ids=lambda f: f.__name__)
def test_varlen_pin(pin):
    pin(oracle)


@pytest.mark.parametrize("pin", _pins.QUANT_PINS, ids=lambda f: f.__name__)
def test_quant_pin(pin):
    pin(oracle)
