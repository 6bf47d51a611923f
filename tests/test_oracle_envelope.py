"""The rank-l envelope (MDBF) form of the fp64 oracle against its pins (CPU
only): the hand-worked example, reduction to the pinned single-profile form
at l = 1, the element-wise envelope formula, linearity in the envelope terms,
and planted mistakes that these pins must catch."""
import json
import os

import numpy as np
import pytest

from oracle import nq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
MODES = {"dense": O.linear_envelope_dense, "factored": O.linear_envelope_factored}


def _hand():
    e = json.load(open(os.path.join(GOLD, "envelope_examples.json")))
    return (np.array(e["x"]), np.array(e["U"], np.int8), np.array(e["V"], np.int8), np.array(e["S1"]),
            np.array(e["g"]), np.array(e["S2"]), np.array(e["y"]), np.array(e["W"]))


def _rand(l, m=6, n=5, r=3, seed=0):
    rng = np.random.default_rng(seed)
    U = rng.choice([-1, 1], size=(m, r)).astype(np.int8)
    V = rng.choice([-1, 1], size=(n, r)).astype(np.int8)
    S1 = rng.integers(-3, 4, size=(l, m)).astype(np.float64)
    S2 = rng.integers(-3, 4, size=(l, n)).astype(np.float64)
    g = rng.integers(1, 4, size=r).astype(np.float64)
    x = rng.integers(-4, 5, size=(2, n)).astype(np.float64)
    return x, U, V, S1, g, S2


def pin_hand_example(f):
    x, U, V, S1, g, S2, y, _ = _hand()
    assert np.array_equal(f(x, U, V, S1, g, S2), y)


def pin_single_term_is_the_base_form(f):
    x, U, V, S1, g, S2 = _rand(1, seed=1)
    assert np.array_equal(f(x, U, V, S1, g, S2), O.linear_dense(x, U, V, S1[0], g, S2[0]))


def pin_elementwise_envelope(f):
    """x W^T with W = (U diag(g) V^T) * (S1^T S2), integer data (exact)."""
    x, U, V, S1, g, S2 = _rand(3, seed=2)
    P = (U.astype(np.float64) * g[None, :]) @ V.astype(np.float64).T
    E = S1.T @ S2
    assert np.array_equal(f(x, U, V, S1, g, S2), x @ (P * E).T)


def pin_linear_in_terms(f):
    x, U, V, S1, g, S2 = _rand(4, seed=3)
    parts = sum(f(x, U, V, S1[i:i + 1], g, S2[i:i + 1]) for i in range(4))
    assert np.array_equal(f(x, U, V, S1, g, S2), parts)


PINS = [pin_hand_example, pin_single_term_is_the_base_form, pin_elementwise_envelope, pin_linear_in_terms]


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, mode):
    pin(MODES[mode])


def test_dense_weight_hand_example():
    _, U, V, S1, g, S2, _, W = _hand()
    assert np.array_equal(O.reconstruct_weight_envelope(U, V, S1, g, S2), W)


def test_rejects_unequal_term_counts():
    x, U, V, S1, g, S2 = _rand(2)
    with pytest.raises(ValueError):
        O.linear_envelope_factored(x, U, V, S1, g, S2[:1])


def _mutants():
    def first_term_only(x, U, V, S1, g, S2):
        return O.linear_dense(x, U, V, np.atleast_2d(S1)[0], g, np.atleast_2d(S2)[0])

    def product_of_profiles(x, U, V, S1, g, S2):    # envelopes multiplied instead of added
        a = np.prod(np.atleast_2d(S1), axis=0)
        b = np.prod(np.atleast_2d(S2), axis=0)
        return O.linear_dense(x, U, V, a, g, b)

    def crossed_terms(x, U, V, S1, g, S2):           # s1 of one term paired with s2 of another
        S1 = np.atleast_2d(S1)
        return O.linear_envelope_factored(x, U, V, S1[::-1], g, S2)

    def summed_profiles(x, U, V, S1, g, S2):         # (sum s1)(sum s2)^T instead of sum of products
        return O.linear_dense(x, U, V, np.atleast_2d(S1).sum(0), g, np.atleast_2d(S2).sum(0))

    return [first_term_only, product_of_profiles, crossed_terms, summed_profiles]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutant):
    caught = 0
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1
