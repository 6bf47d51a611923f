"""GPU: the initialiser (nq_admm_factorize) and magnitude balancing
(nq_balance_scales) against the fp64 oracle on the same seeded inputs.

The iteration decides signs from floating-point values, so the comparison
uses inputs whose sign decisions are far from zero (planted products) for
exact equality of U and V, and compares what is unique elsewhere: W_hat, the
error history, and the sign agreement."""
import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
from oracle import nq_admm as A
from oracle import nq_oracle as O

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def _member(rng, m, r):
    return (rng.choice([-1, 1], size=(m, r)).astype(np.int8), np.abs(rng.standard_normal(m)) + 0.3,
            np.abs(rng.standard_normal(r)) + 0.3)


def _planted(seed, m, n, r):
    rng = np.random.default_rng(seed)
    SA, pA, qA = _member(rng, m, r)
    SB, pB, qB = _member(rng, n, r)
    ZA, ZB = A.compose(SA, pA, qA), A.compose(SB, pB, qB)
    W = (ZA @ ZB.T).astype(np.float32)
    return W, ZA, ZB, SA, SB, rng


def _run(W, A0, B0, rho, iters, K):
    out = nq.admm_factorize(_t(W), _t(A0), _t(B0), rho, iters, K)
    torch.cuda.synchronize()
    return [t.cpu().numpy() if t is not None else None for t in out]


def _what(U, V, s1, g, s2):
    return O.reconstruct_weight(U, V, np.asarray(s1, np.float64), np.asarray(g, np.float64),
                                np.asarray(s2, np.float64))


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - b) / np.linalg.norm(b))


@pytest.mark.parametrize("m,n,r", [(96, 80, 8), (200, 136, 24), (130, 257, 72)])
def test_planted_fixed_point(m, n, r):
    W, ZA, ZB, SA, SB, _ = _planted(m + r, m, n, r)
    print(f"admm fixed point m={m} n={n} r={r}", flush=True)
    U, V, s1, g, s2, err = _run(W, ZA, ZB, 5.0, 3, 4)
    assert np.array_equal(U, SA) and np.array_equal(V, SB)
    assert _rel(_what(U, V, s1, g, s2), W.astype(np.float64)) < 1e-5
    assert np.all(np.abs(err) < 1e-4)


@pytest.mark.parametrize("m,n,r", [(48, 40, 6), (200, 136, 24)])
def test_planted_recovery_matches_oracle(m, n, r):
    W, ZA, ZB, SA, SB, rng = _planted(7 + m, m, n, r)
    A0 = ZA + 0.3 * np.abs(ZA).mean() * rng.standard_normal(ZA.shape)
    B0 = ZB + 0.3 * np.abs(ZB).mean() * rng.standard_normal(ZB.shape)
    A0, B0 = A0.astype(np.float32), B0.astype(np.float32)
    print(f"admm planted recovery m={m} n={n} r={r}", flush=True)
    U, V, s1, g, s2, err = _run(W, A0, B0, 10.0, 40, 20)
    rU, rV, r1, rg, r2, rerr = A.admm_factorize(W.astype(np.float64), A0.astype(np.float64),
                                                B0.astype(np.float64), 10.0, 40, 20)
    assert np.array_equal(U, rU) and np.array_equal(V, rV)
    assert _rel(_what(U, V, s1, g, s2), _what(rU, rV, r1, rg, r2)) < 1e-4
    assert np.max(np.abs(err - rerr)) < 1e-4


@pytest.mark.parametrize("m,n,r", [(200, 136, 24), (64, 64, 64), (300, 190, 40), (520, 390, 130)])
def test_random_weight_matches_oracle(m, n, r):
    rng = np.random.default_rng(100 + m)
    W = rng.standard_normal((m, n)).astype(np.float32)
    A0 = rng.standard_normal((m, r)).astype(np.float32)
    B0 = rng.standard_normal((n, r)).astype(np.float32)
    print(f"admm random m={m} n={n} r={r}", flush=True)
    U, V, s1, g, s2, err = _run(W, A0, B0, 10.0, 4, 8)
    rU, rV, r1, rg, r2, rerr = A.admm_factorize(W.astype(np.float64), A0.astype(np.float64),
                                                B0.astype(np.float64), 10.0, 4, 8)
    # a sign decision may flip only where the latent value is at rounding level
    assert np.mean(U == rU) > 0.999 and np.mean(V == rV) > 0.999
    assert np.max(np.abs(err - rerr) / np.maximum(rerr, 1e-3)) < 2e-3
    assert _rel(_what(U, V, s1, g, s2), _what(rU, rV, r1, rg, r2)) < 2e-3


def test_deterministic():
    rng = np.random.default_rng(3)
    W = _t(rng.standard_normal((120, 90)))
    A0, B0 = _t(rng.standard_normal((120, 16))), _t(rng.standard_normal((90, 16)))
    a = nq.admm_factorize(W, A0, B0, 10.0, 3, 5)
    b = nq.admm_factorize(W, A0, B0, 10.0, 3, 5)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("m,n,r", [(12, 10, 4), (5000, 3000, 300)])
def test_balance_matches_oracle_bitwise(m, n, r):
    rng = np.random.default_rng(m)
    s1 = (37.0 * (np.abs(rng.standard_normal(m)) + 0.1)).astype(np.float32)
    g = (np.abs(rng.standard_normal(r)) + 0.1).astype(np.float32)
    s2 = (0.003 * (np.abs(rng.standard_normal(n)) + 0.1)).astype(np.float32)
    t1, tg, t2 = _t(s1), _t(g), _t(s2)
    nq.balance_scales(t1, tg, t2)
    torch.cuda.synchronize()
    b1, bg, b2 = A.balance_scales(s1, g, s2)
    assert np.array_equal(t1.cpu().numpy(), b1.astype(np.float32))
    assert np.array_equal(tg.cpu().numpy(), bg.astype(np.float32))
    assert np.array_equal(t2.cpu().numpy(), b2.astype(np.float32))


def test_factors_pack_and_run():
    # the initialiser's output is a layer: pack it and run the forward
    W, ZA, ZB, SA, SB, rng = _planted(11, 256, 192, 32)
    U, V, s1, g, s2, _ = nq.admm_factorize(_t(W), _t(ZA), _t(ZB), 5.0, 2, 4, with_err=False)
    nq.balance_scales(s1, g, s2)
    layer = nq.pack(U, V, s1, g, s2)
    x = rng.standard_normal((3, 192)).astype(np.float32)
    y = nq.linear(_t(x), layer, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = x.astype(np.float64) @ W.astype(np.float64).T
    assert _rel(y.cpu().numpy(), ref) < 3e-4
