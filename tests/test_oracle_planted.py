"""Each deliberate mistake built into a copy of the oracle fails at least one
pin, so the pins are sensitive to the mistakes they are meant to catch.

Planted mistakes (see ORACLE_PLANT in oracle/attn_oracle.c):
  1 scale dropped, 2 causal diagonal dropped, 3 window left edge exclusive,
  4 score sign flipped, 5 wrong V row, 6 log base 2 in the LSE,
  7 cache rows aligned top-left instead of at the end of the sequence,
  8 RoPE rotation turned the wrong way, 9 rounding ties away from zero,
  10 backward without the softmax Jacobian's row term,
  11 backward dV magnitude sum doubled, 12 backward dQ magnitude sum without
  its P A term.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.mark.parametrize("plant", [1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12])
def test_planted_mistake_is_caught(plant):
    bad = oracle.load_planted(plant)
    try:
        caught = []
        for pin in ALL_PINS:
            try:
                pin(bad)
            except AssertionError:
                caught.append(pin.__name__)
        assert caught, f"no pin caught planted mistake {plant}"
    finally:
        os.remove(bad.path)
