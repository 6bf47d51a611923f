"""fp64 CPU oracle for the binary low-rank linear layer.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it, and
it imports nothing from the HIP package: the two implementations share no code.

What is computed, and where it comes from
-----------------------------------------
The NanoQuant pages describe the compressed weight as a product of binary
matrices holding only +1 and -1 and of diagonal scaling vectors
(hardwired.dev NanoQuant article, section "Jak NanoQuant funguje"; the
rapidrecap.app summary, "Quantization Technique", names the two binary
matrices U and V and the scaling factors).  The scale placement used here is
the plainest one that the text supports, one diagonal on each side of each
binary factor:

    W_hat = diag(s1) . U . diag(g) . V^T . diag(s2)
    U in {-1,+1}^{m x r},  V in {-1,+1}^{n x r},  s1 in R^m, g in R^r, s2 in R^n

and the layer output for activations x (B x n) is y = x . W_hat^T (B x m), the
orientation of a PyTorch linear layer (m = out features, n = in features).
The method reaches exactly this value, only faster; so the oracle is the
definition written out, with no approximation:

* mode A (``linear_dense``): form W_hat densely in fp64, then multiply;
* mode B (``linear_factored``): the same product evaluated right to left,
  y = s1 * (U (g * (V^T (s2 * x)))), in fp64; used where W_hat is too large.

Storage accounting follows the same article, section "Jak NanoQuant funguje":
an m x n matrix at rank r needs r(m+n) binary values plus the scale
parameters, and the average bits per weight falls below one when r is small
enough (section 'Co znamena "sub-1-bit"').  The scale parameters counted are
the m + n + r entries of s1, g, s2 at ``scale_bits`` each.
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


def linear_factored_rows(x, U_rows, V, s1_rows, g, s2) -> np.ndarray:
    """Mode B restricted to the output features whose rows of U and entries of
    s1 are given: returns y[:, rows] for large layers."""
    return linear_factored(x, U_rows, V, s1_rows, g, s2)


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
    """How many times smaller than an ``original_bits`` model the weights are."""
    return original_bits / bpw
