"""Pins for the fp64 oracle: checks against facts fixed by the pages and by
mathematics, never against the oracle's own formula retyped.

Each pin takes an implementation ``impl(x, U, V, s1, g, s2) -> y`` (x is B x n,
y is B x m) and raises AssertionError when it disagrees with the fact.  The
same pins run against planted mistakes in ``test_oracle_pins.py`` to show that
each plausible mistake fails at least one of them.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import scipy.linalg

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_golden(name: str) -> dict:
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rand_case(rng, m, n, r, B):
    U = (rng.integers(0, 2, size=(m, r)) * 2 - 1).astype(np.int8)
    V = (rng.integers(0, 2, size=(n, r)) * 2 - 1).astype(np.int8)
    s1 = rng.uniform(0.1, 2.0, m)
    g = rng.uniform(0.1, 2.0, r)
    s2 = rng.uniform(0.1, 2.0, n)
    x = rng.standard_normal((B, n))
    return x, U, V, s1, g, s2


def brute_force(x, U, V, s1, g, s2, exact=False):
    """y[b][i] = sum_k sum_j s1_i U_ik g_k V_jk s2_j x_bj, as plain loops
    (Fractions when ``exact``)."""
    conv = (lambda v: Fraction(float(v))) if exact else float
    B, n = len(x), len(x[0])
    m, r = len(U), len(U[0])
    y = [[conv(0) for _ in range(m)] for _ in range(B)]
    for b in range(B):
        for i in range(m):
            acc = conv(0)
            for k in range(r):
                for j in range(n):
                    acc += (conv(s1[i]) * int(U[i][k]) * conv(g[k]) * int(V[j][k])
                            * conv(s2[j]) * conv(x[b][j]))
            y[b][i] = acc
    return y


def _close(a, b, rtol):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    den = max(np.linalg.norm(b), 1e-300)
    err = np.linalg.norm(a - b) / den
    assert err <= rtol, f"relative L2 {err:.3e} > {rtol:.1e}"


# --------------------------------------------------------------------------- pins
def pin_hand_examples(impl):
    for ex in load_golden("hand_examples.json")["examples"]:
        y = impl(np.array(ex["x"]), np.array(ex["U"], np.int8), np.array(ex["V"], np.int8),
                 np.array(ex["s1"]), np.array(ex["g"]), np.array(ex["s2"]))
        assert np.array_equal(np.asarray(y, np.float64), np.array(ex["y"])), (ex["name"], y)


def pin_brute_force(impl):
    rng = np.random.default_rng(1)
    for (m, n, r, B) in [(1, 1, 1, 1), (2, 3, 1, 2), (3, 2, 2, 1), (5, 4, 3, 3), (4, 7, 6, 2), (6, 5, 8, 1)]:
        x, U, V, s1, g, s2 = _rand_case(rng, m, n, r, B)
        _close(impl(x, U, V, s1, g, s2), brute_force(x, U, V, s1, g, s2), 1e-12)


def pin_exact_rationals(impl):
    """Dyadic inputs: every product and sum is exact in fp64, so the result
    must equal the exact rational brute force bit for bit."""
    rng = np.random.default_rng(2)
    for (m, n, r, B) in [(3, 5, 2, 2), (4, 4, 4, 1)]:
        U = (rng.integers(0, 2, size=(m, r)) * 2 - 1).astype(np.int8)
        V = (rng.integers(0, 2, size=(n, r)) * 2 - 1).astype(np.int8)
        s1 = rng.choice([1.0, 2.0, 0.25], m)
        g = rng.choice([1.0, 0.5, 4.0], r)
        s2 = rng.choice([1.0, 2.0, 0.5], n)
        x = rng.integers(-3, 4, size=(B, n)).astype(np.float64)
        ref = brute_force(x, U, V, s1, g, s2, exact=True)
        y = np.asarray(impl(x, U, V, s1, g, s2), np.float64)
        assert [[Fraction(float(v)) for v in row] for row in y] == ref


def pin_hadamard_identity(impl):
    """U = V = H (Sylvester Hadamard, H H^T = n I), s1 = s2 = 1, g = 1/n gives
    W_hat = I, so y = x exactly."""
    rng = np.random.default_rng(3)
    for p in (1, 2, 3, 5):
        n = 2 ** p
        H = scipy.linalg.hadamard(n).astype(np.int8)
        x = rng.integers(-8, 9, size=(2, n)).astype(np.float64)
        y = impl(x, H, H, np.ones(n), np.full(n, 1.0 / n), np.ones(n))
        assert np.array_equal(np.asarray(y, np.float64), x)


def fwht(v: np.ndarray) -> np.ndarray:
    """Fast Walsh-Hadamard transform in Sylvester order (butterfly recurrence),
    O(n log n); equals H_n v for H_n = [[H, H], [H, -H]]."""
    a = np.array(v, dtype=np.float64, copy=True)
    n = a.shape[-1]
    h = 1
    while h < n:
        for i in range(0, n, 2 * h):
            lo = a[..., i:i + h].copy()
            hi = a[..., i + h:i + 2 * h].copy()
            a[..., i:i + h] = lo + hi
            a[..., i + h:i + 2 * h] = lo - hi
        h *= 2
    return a


def pin_walsh_hadamard(impl):
    """U = V = H: y = s1 * H(g * H(s2 * x)) (H is symmetric), computed by the
    fast transform instead of any matrix product."""
    rng = np.random.default_rng(4)
    for n in (4, 16, 64):
        H = scipy.linalg.hadamard(n).astype(np.int8)
        s1, g, s2 = rng.uniform(0.1, 2, n), rng.uniform(0.1, 2, n), rng.uniform(0.1, 2, n)
        x = rng.standard_normal((3, n))
        ref = s1 * fwht(g * fwht(s2 * x))
        _close(impl(x, H, H, s1, g, s2), ref, 1e-13)


def pin_rank_one(impl):
    """r = 1: y = g1 <v, s2*x> (s1*u)."""
    rng = np.random.default_rng(5)
    m, n = 7, 5
    x, U, V, s1, g, s2 = _rand_case(rng, m, n, 1, 3)
    u, v = U[:, 0].astype(np.float64), V[:, 0].astype(np.float64)
    ref = np.stack([g[0] * float(np.dot(v, s2 * xb)) * (s1 * u) for xb in x])
    _close(impl(x, U, V, s1, g, s2), ref, 1e-13)


def pin_sign_flip(impl):
    """Negating column k of both U and V leaves W_hat unchanged, since
    (-a)(-b) = ab exactly."""
    rng = np.random.default_rng(6)
    x, U, V, s1, g, s2 = _rand_case(rng, 6, 9, 5, 2)
    y0 = np.asarray(impl(x, U, V, s1, g, s2))
    for k in range(5):
        U2, V2 = U.copy(), V.copy()
        U2[:, k] *= -1
        V2[:, k] *= -1
        _close(impl(x, U2, V2, s1, g, s2), y0, 1e-14)
    # flipping only one side must change the answer (it negates one rank-1 term)
    U3 = U.copy()
    U3[:, 0] *= -1
    assert np.linalg.norm(np.asarray(impl(x, U3, V, s1, g, s2)) - y0) > 1e-6 * np.linalg.norm(y0)


def pin_g_sign_absorption(impl):
    """Negating column k of U together with g_k leaves W_hat unchanged."""
    rng = np.random.default_rng(7)
    x, U, V, s1, g, s2 = _rand_case(rng, 5, 6, 4, 2)
    y0 = np.asarray(impl(x, U, V, s1, g, s2))
    U2, g2 = U.copy(), g.copy()
    U2[:, 2] *= -1
    g2[2] *= -1
    _close(impl(x, U2, V, s1, g2, s2), y0, 1e-14)


def pin_rank_permutation(impl):
    """Permuting the rank index jointly in U, V and g leaves W_hat unchanged."""
    rng = np.random.default_rng(8)
    x, U, V, s1, g, s2 = _rand_case(rng, 6, 7, 5, 2)
    perm = rng.permutation(5)
    _close(impl(x, U[:, perm], V[:, perm], s1, g[perm], s2), impl(x, U, V, s1, g, s2), 1e-14)


def pin_linearity_and_rows(impl):
    """y(2^a x) = 2^a y(x) exactly, and each batch row is computed on its own."""
    rng = np.random.default_rng(9)
    x, U, V, s1, g, s2 = _rand_case(rng, 5, 6, 3, 4)
    y = np.asarray(impl(x, U, V, s1, g, s2))
    assert np.array_equal(np.asarray(impl(8.0 * x, U, V, s1, g, s2)), 8.0 * y)
    for b in range(4):
        _close(impl(x[b:b + 1], U, V, s1, g, s2)[0], y[b], 1e-14)


PINS = [pin_hand_examples, pin_brute_force, pin_exact_rationals, pin_hadamard_identity,
        pin_walsh_hadamard, pin_rank_one, pin_sign_flip, pin_g_sign_absorption,
        pin_rank_permutation, pin_linearity_and_rows]
