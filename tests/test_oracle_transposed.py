"""The transposed product of the fp64 oracle against its pins (CPU only):
the hand-worked example, adjointness with the pinned forward, the Hadamard
identity, and planted mistakes that these pins must catch."""
import json
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import nq_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
MODES = {"dense": O.linear_transposed_dense, "factored": O.linear_transposed_factored}


def _hand():
    ex = {e["name"]: e for e in json.load(open(os.path.join(GOLD, "hand_examples.json")))["examples"]}
    t = json.load(open(os.path.join(GOLD, "transposed_examples.json")))
    L = ex[t["layer"]]
    return (np.array(t["dy"]), np.array(L["U"], np.int8), np.array(L["V"], np.int8), np.array(L["s1"]),
            np.array(L["g"]), np.array(L["s2"]), np.array(t["dx"]))


def pin_hand_example(f):
    dy, U, V, s1, g, s2, dx = _hand()
    assert np.array_equal(f(dy, U, V, s1, g, s2), dx)


def pin_adjoint_of_forward(f):
    """<W x, dy> = <x, W^T dy> with the forward oracle, on integer data (exact)."""
    rng = np.random.default_rng(7)
    for (m, n, r) in [(5, 3, 2), (3, 7, 4), (16, 16, 5)]:
        U = rng.choice([-1, 1], size=(m, r)).astype(np.int8)
        V = rng.choice([-1, 1], size=(n, r)).astype(np.int8)
        s1, g, s2 = (rng.integers(1, 5, size=k).astype(np.float64) for k in (m, r, n))
        x = rng.integers(-4, 5, size=(3, n)).astype(np.float64)
        dy = rng.integers(-4, 5, size=(3, m)).astype(np.float64)
        lhs = np.sum(O.linear_dense(x, U, V, s1, g, s2) * dy, axis=1)
        rhs = np.sum(x * f(dy, U, V, s1, g, s2), axis=1)
        assert np.array_equal(lhs, rhs)


def pin_unit_rows_give_rows_of_w(f):
    """dy = e_i gives row i of the dense hand-worked W."""
    ex = json.load(open(os.path.join(GOLD, "hand_examples.json")))["examples"][1]
    W = np.array(ex["W"])
    dy = np.eye(W.shape[0])
    assert np.array_equal(f(dy, np.array(ex["U"], np.int8), np.array(ex["V"], np.int8), ex["s1"], ex["g"],
                            ex["s2"]), W)


def pin_hadamard_identity(f):
    n = 16
    H = scipy.linalg.hadamard(n).astype(np.int8)
    dy = np.arange(2 * n, dtype=np.float64).reshape(2, n) - 7
    assert np.array_equal(f(dy, H, H, np.ones(n), np.full(n, 1.0 / n), np.ones(n)), dy)


PINS = [pin_hand_example, pin_adjoint_of_forward, pin_unit_rows_give_rows_of_w, pin_hadamard_identity]


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(pin, mode):
    pin(MODES[mode])


def test_swapped_roles_are_the_forward_of_the_transpose():
    """W_hat^T is the layer with U <-> V and s1 <-> s2 (what the GPU path packs)."""
    rng = np.random.default_rng(3)
    m, n, r = 9, 13, 6
    U = rng.choice([-1, 1], size=(m, r)).astype(np.int8)
    V = rng.choice([-1, 1], size=(n, r)).astype(np.int8)
    s1, g, s2 = (rng.random(k) + 0.5 for k in (m, r, n))
    dy = rng.standard_normal((4, m))
    a = O.linear_transposed_factored(dy, U, V, s1, g, s2)
    b = O.linear_factored(dy, V, U, s2, g, s1)
    assert np.allclose(a, b, rtol=1e-13, atol=0)


def _mutants():
    f64 = lambda a: np.asarray(a, np.float64)

    def forward_instead(dy, U, V, s1, g, s2):          # no transpose: rows of W^T used as W
        W = O.reconstruct_weight(U, V, s1, g, s2)
        return f64(dy) @ np.resize(W.T, (W.shape[0], W.shape[1]))

    def scales_not_swapped(dy, U, V, s1, g, s2):       # s1 applied at the output side
        return O.linear_factored(dy, V, U, np.resize(f64(s1), len(s2)), g, np.resize(f64(s2), len(s1)))

    def dropped_g(dy, U, V, s1, g, s2):
        return O.linear_transposed_factored(dy, U, V, s1, np.ones_like(f64(g)), s2)

    def sign_flipped_U(dy, U, V, s1, g, s2):
        return O.linear_transposed_factored(dy, -np.asarray(U), V, s1, g, s2)

    return [forward_instead, scales_not_swapped, dropped_g, sign_flipped_U]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mutant):
    caught = 0
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1
