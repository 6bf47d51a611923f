"""fp64 CPU oracle for the binary low-rank linear layer.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it, and
it imports nothing from the HIP package: the two implementations share no code.

What is computed, and where it comes from
-----------------------------------------
Sources: hardwired.dev NanoQuant article, section "Jak NanoQuant funguje"
(the weight is factored into +-1 matrices and diagonal scale vectors; the
storage rule in bits); rapidrecap.app summary, section "Quantization
Technique" (the two sign matrices are named U and V).  The articles fix the
ingredients but not where each diagonal sits; this oracle takes one diagonal
on each side of each sign factor, the plainest placement they allow:

    W_hat = diag(s1) . U . diag(g) . V^T . diag(s2)
    U in {-1,+1}^{m x r},  V in {-1,+1}^{n x r},  s1 in R^m, g in R^r, s2 in R^n

For activations x (B x n) the layer output is y = x . W_hat^T (B x m), the
orientation of a PyTorch linear layer (m = out features, n = in features).
The fast path computes exactly this value in another order, so the oracle is
the definition itself, with no approximation:

* mode A (``linear_dense``): form W_hat densely in fp64, then multiply;
* mode B (``linear_factored``): the same product evaluated right to left,
  y = s1 * (U (g * (V^T (s2 * x)))), in fp64; used where W_hat is too large.

The backward product through the layer (same article, section "Trikrokovy
pipeline", step 3: the factors are refined block by block by propagating
gradients through the binarised layer) needs W_hat^T applied to an output
gradient: for dy (B x m), dx = dy . W_hat (B x n), i.e. W_hat^T dy row by row:

* ``linear_transposed_dense``: W_hat formed densely, dx = dy W_hat;
* ``linear_transposed_factored``: dx = s2 * (V (g * (U^T (s1 * dy)))).

Format variants (same article, section "Kontext: co existuje kolem"): DBF
factors a weight into two binary matrices with diagonal scaling, so every
rank component carries the same magnitude profile; that is the form above
(the profile s1 s2^T, weighted by g).  MDBF replaces that single profile by
an envelope of rank l.  Plainest reading: the sign product U diag(g) V^T is
modulated element by element by E = sum_l s1^(l) s2^(l)^T, i.e.

    W_hat = sum_l diag(s1^(l)) . U . diag(g) . V^T . diag(s2^(l)),

with l pairs of scale vectors sharing U, V and g (``reconstruct_weight_envelope``,
``linear_envelope_dense``, ``linear_envelope_factored``); l = 1 is the form above.

Storage (same article and section, plus section 'Co znamena "sub-1-bit"'):
a rank-r factorisation of an m x n matrix stores r(m+n) sign bits; the scale
parameters counted here are the m + n + r entries of s1, g, s2 at
``scale_bits`` each, so bits per weight = (r(m+n) + scale_bits(m+n+r)) / (mn),
which is below 1 when r is small.  ``compression_ratio`` is the size of a
16-bit dense weight over the stored size (section "Cisla" quotes 25.8x for
Llama2-70B, 138.04 GB against 5.35 GB).
"""
from __future__ import annotations

import math

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def _check_signs(M: np.ndarray, name: str) -> None:
    if not np.all((M == 1) | (M == -1)):
        raise ValueError(f"{name} must hold only +1 and -1")


def reconstruct_weight(U, V, s1, g, s2) -> np.ndarray:
    """W_hat = diag(s1) U diag(g) V^T diag(s2), dense, fp64, shape (m, n)."""
    U = np.asarray(U)
    V = np.asarray(V)
    _check_signs(U, "U")
    _check_signs(V, "V")
    left = _f64(s1)[:, None] * _f64(U)          # diag(s1) U        (m x r)
    mid = _f64(g)[:, None] * _f64(V).T           # diag(g) V^T       (r x n)
    return (left @ mid) * _f64(s2)[None, :]      # ... diag(s2)      (m x n)


def linear_dense(x, U, V, s1, g, s2) -> np.ndarray:
    """Mode A: y = x W_hat^T with W_hat formed densely.  x is (B, n); y is (B, m)."""
    W = reconstruct_weight(U, V, s1, g, s2)
    return _f64(x) @ W.T


def linear_factored(x, U, V, s1, g, s2) -> np.ndarray:
    """Mode B: y = s1 * (U (g * (V^T (s2 * x)))), row by row of x, in fp64."""
    U = np.asarray(U)
    V = np.asarray(V)
    _check_signs(U, "U")
    _check_signs(V, "V")
    xs = _f64(x) * _f64(s2)[None, :]             # s2 * x            (B x n)
    t = xs @ _f64(V)                             # V^T (s2 x)        (B x r)
    t = t * _f64(g)[None, :]                     # g * t
    z = t @ _f64(U).T                            # U t'              (B x m)
    return z * _f64(s1)[None, :]                 # s1 * z


def linear_transposed_dense(dy, U, V, s1, g, s2) -> np.ndarray:
    """dx = dy W_hat with W_hat formed densely.  dy is (B, m); dx is (B, n)."""
    W = reconstruct_weight(U, V, s1, g, s2)
    return _f64(dy) @ W


def linear_transposed_factored(dy, U, V, s1, g, s2) -> np.ndarray:
    """dx = s2 * (V (g * (U^T (s1 * dy)))), row by row of dy, in fp64."""
    U = np.asarray(U)
    V = np.asarray(V)
    _check_signs(U, "U")
    _check_signs(V, "V")
    ds = _f64(dy) * _f64(s1)[None, :]            # s1 * dy           (B x m)
    t = ds @ _f64(U)                             # U^T (s1 dy)       (B x r)
    t = t * _f64(g)[None, :]                     # g * t
    z = t @ _f64(V).T                            # V t'              (B x n)
    return z * _f64(s2)[None, :]                 # s2 * z


def reconstruct_weight_envelope(U, V, S1, g, S2) -> np.ndarray:
    """W_hat = sum_l diag(S1[l]) U diag(g) V^T diag(S2[l]); S1 is (l, m), S2 (l, n)."""
    S1 = np.atleast_2d(_f64(S1))
    S2 = np.atleast_2d(_f64(S2))
    if S1.shape[0] != S2.shape[0]:
        raise ValueError("S1 and S2 must hold the same number of envelope terms")
    W = np.zeros((S1.shape[1], S2.shape[1]))
    for a, b in zip(S1, S2):
        W += reconstruct_weight(U, V, a, g, b)
    return W


def linear_envelope_dense(x, U, V, S1, g, S2) -> np.ndarray:
    """y = x W_hat^T for the rank-l envelope form, W_hat formed densely."""
    return _f64(x) @ reconstruct_weight_envelope(U, V, S1, g, S2).T


def linear_envelope_factored(x, U, V, S1, g, S2) -> np.ndarray:
    """y = sum_l S1[l] * (U (g * (V^T (S2[l] * x)))), in fp64."""
    S1 = np.atleast_2d(_f64(S1))
    S2 = np.atleast_2d(_f64(S2))
    if S1.shape[0] != S2.shape[0]:
        raise ValueError("S1 and S2 must hold the same number of envelope terms")
    y = np.zeros((np.atleast_2d(x).shape[0], S1.shape[1]))
    for a, b in zip(S1, S2):
        y += linear_factored(x, U, V, a, g, b)
    return y


def bits_per_weight(m: int, n: int, r: int, scale_bits: int = 16) -> float:
    """Average stored bits per original weight: r(m+n) sign bits plus
    (m+n+r) scales of ``scale_bits`` bits, over m*n weights."""
    if m <= 0 or n <= 0 or r < 0 or scale_bits < 0:
        raise ValueError("dimensions must be positive")
    return (r * (m + n) + scale_bits * (m + n + r)) / (m * n)


def rank_for_bits(m: int, n: int, bpw: float, scale_bits: int = 16) -> int:
    """Largest rank r >= 1 whose bits_per_weight is at most ``bpw``; 0 if none.

    bits_per_weight is increasing in r, so the answer is the floor of the
    root of bpw(r) = target, found here by direct search from that estimate
    (no closed form is trusted on its own)."""
    if bits_per_weight(m, n, 1, scale_bits) > bpw:
        return 0
    r = max(1, int(math.floor((bpw * m * n - scale_bits * (m + n)) / (m + n + scale_bits))))
    while r > 1 and bits_per_weight(m, n, r, scale_bits) > bpw:
        r -= 1
    while bits_per_weight(m, n, r + 1, scale_bits) <= bpw:
        r += 1
    return r


def compression_ratio(bpw: float, original_bits: int = 16) -> float:
    """How many times smaller than a dense ``original_bits``-per-weight matrix
    the stored factorisation is, given its average bits per weight."""
    if not bpw > 0:
        raise ValueError("bits per weight must be positive")
    return original_bits / bpw


def stored_bytes(m: int, n: int, r: int, scale_bits: int = 16) -> float:
    """Bytes of one stored factorisation (sign bits plus scales, no padding)."""
    return bits_per_weight(m, n, r, scale_bits) * m * n / 8.0
