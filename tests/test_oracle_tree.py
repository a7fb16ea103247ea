"""Pins of the oracle's token-tree verification (tests/tree_pins.py): hand-worked forced trees, a
chain equal to the linear draft, the greedy walk against numpy, losslessness by chi-square of the
emitted tokens given their prefix, and the Philox blocks a tree's decisions take."""
import numpy as np
import pytest

import tree_pins
from oracle import oracle
from workloads import offsets_from_depths


@pytest.mark.parametrize("pin", tree_pins.ALL, ids=lambda f: f.__name__)
def test_tree_pin(pin):
    assert pin()


def test_lossless_at_another_temperature():
    assert tree_pins.pin_lossless(T=0.7, calls=24)


def test_empty_trees_draw_one_target_token():
    """A request with no nodes draws its one token from the root's target distribution, as the
    linear rule does at K = 0."""
    rng = np.random.default_rng(4)
    B, V = 32, 50
    target = rng.standard_normal((B, V)).astype(np.float32)
    cu = offsets_from_depths(np.zeros(B, dtype=int))
    empty = np.zeros(0, dtype=np.int32)
    tree = oracle.verify_tree(target, np.zeros((0, V), np.float32), empty, empty, cu, 1.0, 5)
    lin = oracle.verify(target, np.zeros((0, V), np.float32), empty, cu, 1.0, 5)
    assert np.array_equal(tree["out_tokens"], lin["out_tokens"]) and (tree["accepted_len"] == 0).all()


def test_argument_errors():
    t = np.zeros((2, 4), np.float32)
    one = np.zeros(1, dtype=np.int32)
    with pytest.raises(ValueError):
        oracle.verify_tree(t, None, one, -one, offsets_from_depths([1]), 1.0, 0)  # T > 0 without draft rows
    with pytest.raises(ValueError):
        oracle.verify_tree(t, None, one, -one, offsets_from_depths([1]), -1.0, 0)
