"""The initialiser's fp64 oracle (oracle/nq_admm.py) against pins that do not
come from itself (CPU only): the projection against exhaustive enumeration of
the sign patterns and against numpy's SVD, the closed-form least-squares step
against numpy's least-squares solver on the stacked system, the planted
product as an exact fixed point and as a point of attraction, the balancing's
bitwise invariance, and planted mistakes that these pins must catch."""
import itertools

import numpy as np
import pytest

from oracle import nq_admm as A
from oracle import nq_oracle as O


def _member(rng, m, r):
    S = rng.choice([-1, 1], size=(m, r)).astype(np.int8)
    return S, np.abs(rng.standard_normal(m)) + 0.3, np.abs(rng.standard_normal(r)) + 0.3


def _planted(seed=0, m=48, n=40, r=6):
    rng = np.random.default_rng(seed)
    SA, pA, qA = _member(rng, m, r)
    SB, pB, qB = _member(rng, n, r)
    ZA, ZB = A.compose(SA, pA, qA), A.compose(SB, pB, qB)
    return ZA @ ZB.T, ZA, ZB, SA, SB


# ---------------------------------------------------------------- projection
def pin_projection_keeps_members(project):
    rng = np.random.default_rng(1)
    S, p, q = _member(rng, 7, 5)
    Y = A.compose(S, p, q)
    S2, p2, q2 = project(Y, 3)
    assert np.array_equal(S2, S)
    assert np.allclose(A.compose(S2, p2, q2), Y, rtol=1e-12, atol=1e-12)


def pin_projection_magnitude_is_leading_singular_pair(project):
    rng = np.random.default_rng(2)
    Y = rng.standard_normal((9, 6))
    _, p, q = project(Y, 400)
    u, s, vt = np.linalg.svd(np.abs(Y))
    ref = s[0] * np.outer(np.abs(u[:, 0]), np.abs(vt[0]))
    assert np.allclose(np.outer(p, q), ref, rtol=1e-9, atol=1e-12)


def pin_projection_beats_every_sign_pattern(project):
    # For each of the 2^6 sign patterns S', the best rank-1 magnitude (not even
    # restricted to p, q >= 0) leaves at least ||Y||^2 - sigma_1(S' . Y)^2; the
    # projection's error must not exceed any of these lower bounds.
    rng = np.random.default_rng(3)
    Y = rng.standard_normal((2, 3))
    S, p, q = project(Y, 300)
    err = np.sum((Y - A.compose(S, p, q)) ** 2)
    for bits in itertools.product([-1, 1], repeat=6):
        Sp = np.array(bits, dtype=np.float64).reshape(2, 3)
        bound = np.sum(Y ** 2) - np.linalg.svd(Sp * Y, compute_uv=False)[0] ** 2
        assert err <= bound + 1e-12


def pin_projection_sign_of_zero(project):
    S, _, _ = project(np.zeros((2, 2)), 2)
    assert np.all(S == 1)


@pytest.mark.parametrize("pin", [pin_projection_keeps_members, pin_projection_magnitude_is_leading_singular_pair,
                                 pin_projection_beats_every_sign_pattern, pin_projection_sign_of_zero])
def test_projection_pins(pin):
    pin(A.project)


# ---------------------------------------------------------------- least squares
def pin_latent_update_is_least_squares(update):
    rng = np.random.default_rng(4)
    m, n, r, rho = 7, 6, 3, 0.7
    W, Bc = rng.standard_normal((m, n)), rng.standard_normal((n, r))
    Z, L = rng.standard_normal((m, r)), rng.standard_normal((m, r))
    # minimise ||W - A Bc^T||^2 + rho ||A - (Z - L)||^2 as one stacked
    # least-squares problem: A [Bc^T, sqrt(rho) I] ~ [W, sqrt(rho) (Z - L)]
    M = np.vstack([Bc, np.sqrt(rho) * np.eye(r)])
    R = np.hstack([W, np.sqrt(rho) * (Z - L)])
    ref = np.linalg.lstsq(M, R.T, rcond=None)[0].T
    assert np.allclose(update(W, Bc, Z, L, rho), ref, rtol=1e-10, atol=1e-12)


def test_latent_update_is_least_squares():
    pin_latent_update_is_least_squares(A.latent_update)


# ---------------------------------------------------------------- the iteration
def test_planted_product_is_a_fixed_point():
    W, ZA, ZB, SA, SB = _planted()
    U, V, s1, g, s2, err = A.admm_factorize(W, ZA, ZB, 5.0, 4, 3)
    assert np.array_equal(U, SA) and np.array_equal(V, SB)
    assert np.allclose(O.reconstruct_weight(U, V, s1, g, s2), W, rtol=1e-12, atol=1e-10)
    assert np.all(err < 1e-24)


def test_planted_product_attracts_a_perturbed_start():
    W, ZA, ZB, SA, SB = _planted(seed=5)
    rng = np.random.default_rng(6)
    A0 = ZA + 0.3 * np.abs(ZA).mean() * rng.standard_normal(ZA.shape)
    B0 = ZB + 0.3 * np.abs(ZB).mean() * rng.standard_normal(ZB.shape)
    U, V, s1, g, s2, err = A.admm_factorize(W, A0, B0, 10.0, 40, 20)
    assert err[-1] < 1e-3 * err[0]
    assert np.array_equal(U, SA) and np.array_equal(V, SB)


def test_admm_improves_a_random_start():
    rng = np.random.default_rng(7)
    W = rng.standard_normal((40, 32))
    U, V, s1, g, s2, err = A.admm_factorize(W, rng.standard_normal((40, 8)), rng.standard_normal((32, 8)), 10.0,
                                            10, 10)
    assert err[-1] < 0.25 * err[0] and err[-1] < 1.2
    assert set(np.unique(U)) <= {-1, 1} and set(np.unique(V)) <= {-1, 1}
    assert np.all(s1 >= 0) and np.all(g >= 0) and np.all(s2 >= 0)
    # err is the definition: ||W - W_hat||^2 / ||W||^2 with W_hat from the outputs
    What = O.reconstruct_weight(U, V, s1, g, s2)
    assert abs(np.sum((W - What) ** 2) / np.sum(W ** 2) - err[-1]) < 1e-12


# ---------------------------------------------------------------- balancing
def test_balancing_is_bitwise_invariant_and_balanced():
    rng = np.random.default_rng(8)
    U = rng.choice([-1, 1], size=(12, 4)).astype(np.int8)
    V = rng.choice([-1, 1], size=(10, 4)).astype(np.int8)
    s1, g, s2 = 37.0 * (np.abs(rng.standard_normal(12)) + 0.1), np.abs(rng.standard_normal(4)) + 0.1, \
        0.003 * (np.abs(rng.standard_normal(10)) + 0.1)
    b1, bg, b2 = A.balance_scales(s1, g, s2)
    assert np.array_equal(O.reconstruct_weight(U, V, b1, bg, b2), O.reconstruct_weight(U, V, s1, g, s2))
    for v in (b1, b2):
        rms = np.sqrt(np.mean(v ** 2))
        assert 1.0 <= rms < 2.0
    assert A.balance_exponent(np.zeros(3)) == 1.0


# ---------------------------------------------------------------- planted mistakes
def _proj_no_abs(Y, K):  # magnitude fit on Y instead of |Y|
    Y = np.asarray(Y, np.float64)
    S = np.where(Y >= 0, 1, -1).astype(np.int8)
    q = np.full(Y.shape[1], 1 / np.sqrt(Y.shape[1]))
    sigma = 0.0
    for _ in range(K):
        p = Y @ q
        p /= np.linalg.norm(p)
        q = Y.T @ p
        sigma = np.linalg.norm(q)
        q /= sigma
    return S, p * np.sqrt(sigma), q * np.sqrt(sigma)


def _proj_sign_of_zero_negative(Y, K):
    S, p, q = A.project(Y, K)
    return np.where(np.asarray(Y) > 0, 1, -1).astype(np.int8), p, q


def _update_wrong_penalty_side(W, Bc, Z, L, rho):  # Z + L instead of Z - L
    return A.latent_update(W, Bc, Z, -np.asarray(L), rho)


def _update_gram_without_rho(W, Bc, Z, L, rho):
    W, Bc, Z, L = (np.asarray(t, np.float64) for t in (W, Bc, Z, L))
    R = W @ Bc + rho * (Z - L)
    return np.linalg.solve(Bc.T @ Bc, R.T).T


@pytest.mark.parametrize("mutant,pins", [
    (_proj_no_abs, [pin_projection_magnitude_is_leading_singular_pair, pin_projection_beats_every_sign_pattern]),
    (_proj_sign_of_zero_negative, [pin_projection_sign_of_zero]),
])
def test_projection_mutants_are_caught(mutant, pins):
    caught = 0
    for pin in pins:
        try:
            pin(mutant)
        except (AssertionError, FloatingPointError, ValueError, np.linalg.LinAlgError):
            caught += 1
    assert caught >= 1


@pytest.mark.parametrize("mutant", [_update_wrong_penalty_side, _update_gram_without_rho])
def test_update_mutants_are_caught(mutant):
    with pytest.raises(AssertionError):
        pin_latent_update_is_least_squares(mutant)
