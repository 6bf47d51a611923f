"""fp64 CPU oracle for the initialiser of the binary factorisation.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it, and
it imports nothing from the HIP package.

Source: hardwired.dev NanoQuant article, section "Trikrokovy pipeline",
step 2 (LB-ADMM) and the paragraph after it.  There the initialiser is an
ADMM method for the discrete choice of sign matrices and scales that best
reproduce a weight: each iteration solves for the real-valued part by least
squares in closed form and maps onto the +-1 set by taking signs; a
magnitude-balancing step on the scale factors follows it.  The article gives
no equation, no penalty parameter and no iteration count.  Plainest reading (identity Hessian: no
calibration data here, so every weight counts the same):

    minimise ||W - A B^T||_F^2  over A (m x r), B (n x r)
    subject to A, B in C = { diag(p) S diag(q) : S in {-1,+1}, p, q >= 0 }

so that A B^T = diag(p_A) S_A diag(q_A q_B) S_B^T diag(p_B) is exactly the
stored form W_hat = diag(s1) U diag(g) V^T diag(s2) with U = S_A, V = S_B,
s1 = p_A, g = q_A * q_B, s2 = p_B.  ADMM splits each factor into a continuous
latent copy (A, B) and its constrained copy (Z_A, Z_B) with scaled duals
(L_A, L_B) and penalty rho:

    A   <- (W B + rho (Z_A - L_A)) (B^T B + rho I)^-1       least squares, closed form
    B   <- (W^T A + rho (Z_B - L_B)) (A^T A + rho I)^-1
    Z_A <- proj_C(A + L_A),  Z_B <- proj_C(B + L_B)          sign projection
    L_A <- L_A + A - Z_A,    L_B <- L_B + B - Z_B

proj_C(Y) is the exact Euclidean projection onto C: for any p, q >= 0 the best
S is sign(Y) (entry by entry), and then ||Y - S . pq^T|| = || |Y| - p q^T ||, so
(p, q) is the leading singular pair of the non-negative |Y| (non-negative by
Perron-Frobenius), found here by K power steps started from the constant
vector.  sign(0) is taken as +1 (entries must be exactly +-1).

Magnitude balancing (same section, the paragraph after step 2): the scale
vectors are rescaled by powers of two, s1 * c, s2 * d, g / (c d), with c and d
chosen so that the root-mean-square of s1 and of s2 lies in [1, 2).  A power of
two changes no significand, so W_hat is unchanged bit for bit.
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def project(Y, power_iters):
    """proj_C(Y): (S int8 +-1, p >= 0, q >= 0) with diag(p) S diag(q) the
    projection of Y onto the sign-times-rank-1-magnitude set.  p, q come from
    `power_iters` power steps on |Y| from q = 1/sqrt(r) (r = columns)."""
    Y = _f64(Y)
    S = np.where(Y >= 0.0, 1, -1).astype(np.int8)
    M = np.abs(Y)
    r = Y.shape[1]
    q = np.full(r, 1.0 / np.sqrt(r))
    p = np.zeros(Y.shape[0])
    sigma = 0.0
    for _ in range(power_iters):
        p = M @ q
        nrm = np.linalg.norm(p)
        if nrm > 0.0:
            p = p / nrm
        q = M.T @ p
        sigma = np.linalg.norm(q)
        if sigma > 0.0:
            q = q / sigma
    root = np.sqrt(sigma)
    return S, p * root, q * root


def compose(S, p, q):
    """diag(p) S diag(q) as a dense fp64 matrix."""
    return _f64(p)[:, None] * _f64(S) * _f64(q)[None, :]


def latent_update(W, Bc, Z, L, rho):
    """argmin_A ||W - A Bc^T||^2 + rho ||A - (Z - L)||^2 in closed form:
    A = (W Bc + rho (Z - L)) (Bc^T Bc + rho I)^-1."""
    W, Bc, Z, L = _f64(W), _f64(Bc), _f64(Z), _f64(L)
    r = Bc.shape[1]
    G = Bc.T @ Bc + rho * np.eye(r)
    R = W @ Bc + rho * (Z - L)
    return np.linalg.solve(G, R.T).T


def admm_factorize(W, A0, B0, rho, iters, power_iters):
    """The initialiser above: `iters` ADMM steps from the latent factors A0,
    B0 (Z and the duals start at proj_C(A0), proj_C(B0) and 0).  Returns
    (U, V, s1, g, s2, err) with err[t] = ||W - Z_A Z_B^T||_F^2 / ||W||_F^2
    after t steps (err[0]: the starting point)."""
    W = _f64(W)
    A, B = _f64(A0), _f64(B0)
    SA, pA, qA = project(A, power_iters)
    SB, pB, qB = project(B, power_iters)
    ZA, ZB = compose(SA, pA, qA), compose(SB, pB, qB)
    LA, LB = np.zeros_like(A), np.zeros_like(B)
    w2 = float(np.sum(W * W))
    err = [float(np.sum((W - ZA @ ZB.T) ** 2)) / w2]
    for _ in range(iters):
        A = latent_update(W, B, ZA, LA, rho)
        B = latent_update(W.T, A, ZB, LB, rho)
        SA, pA, qA = project(A + LA, power_iters)
        SB, pB, qB = project(B + LB, power_iters)
        ZA, ZB = compose(SA, pA, qA), compose(SB, pB, qB)
        LA = LA + A - ZA
        LB = LB + B - ZB
        err.append(float(np.sum((W - ZA @ ZB.T) ** 2)) / w2)
    return SA, SB, pA, qA * qB, pB, np.array(err)


def balance_exponent(v):
    """The power of two c with rms(v) * c in [1, 2) (1 for a zero vector)."""
    rms = float(np.sqrt(np.mean(_f64(v) ** 2)))
    if not rms > 0.0 or not np.isfinite(rms):
        return 1.0
    _, e = np.frexp(rms)  # rms = f 2^e, f in [0.5, 1)
    return float(np.ldexp(1.0, 1 - int(e)))


def balance_scales(s1, g, s2):
    """Magnitude balancing: (s1 c, g / (c d), s2 d) with c, d powers of two
    putting rms(s1 c) and rms(s2 d) in [1, 2)."""
    c, d = balance_exponent(s1), balance_exponent(s2)
    return _f64(s1) * c, _f64(g) / (c * d), _f64(s2) * d
