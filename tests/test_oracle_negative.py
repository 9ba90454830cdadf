"""Negative controls: builds of the oracle with one planted mistake each must fail a pin.

This shows that the pins have the power to catch the plausible mistakes listed
in the oracle's planted-mistake catalogue (a dropped term, a wrong sign, a
wrong index or operand, a wrong comparison, a missing step).  The mistakes are
compiled into separate copies of the oracle in a temporary directory; the real
oracle is untouched.
"""
import numpy as np
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def plant_dir(tmp_path_factory):
    return str(tmp_path_factory.mktemp("plants"))


@pytest.mark.parametrize("name", sorted(oracle.PLANTS))
def test_planted_mistake_is_caught(name, plant_dir):
    o = oracle.load_planted(name, plant_dir)
    assert o.planted == oracle.PLANTS[name]
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, IndexError) as e:  # a pin failing is what we want
            caught.append((pin.__name__, type(e).__name__))
            break
    assert caught, f"planted mistake {name!r} passed every pin"


def test_resample_from_p_matches_the_lessons_prediction(plant_dir):
    """The lesson's "Break It" section predicts that drawing from p on rejection gives
    min(p, q) + (1 - alpha) p instead of p; on the page-4 toy vectors that is far from p."""
    o = oracle.load_planted("resample_from_p", plant_dir)
    g = oracle_pins.golden("prep_demo.json")
    p = np.array(g["p"], np.float32)
    q = np.array(g["q"], np.float32)
    counts, _ = oracle_pins._first_token_stats(o, p, q, 1, g["trials"], seed=42)
    alpha = float(np.minimum(p, q).astype(np.float64).sum())
    predicted = np.minimum(p, q).astype(np.float64) + (1 - alpha) * p.astype(np.float64)
    assert oracle_pins._tv(counts, predicted) < 0.005
    assert oracle_pins._tv(counts, p) > 0.04
