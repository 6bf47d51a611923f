"""GPU parity of the large-batch (prefill) path: both sign-matrix products as
fp16 MFMA GEMMs with exact +-1 operands, against the fp64 oracle.

Tolerance: the activation operand of each GEMM is rounded once to fp16 after a
power-of-two row scale (unit roundoff 2^-11, RMS relative error ~ 2^-11/sqrt(3)
= 2.8e-4 per rounding, independent across terms); two roundings give ~4e-4
relative L2 on fp32 outputs, bounded here by 1e-3."""
import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
import synth
from oracle import nq_oracle as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

TOL32 = 1e-3


@pytest.mark.parametrize("m,n,r", [(256, 256, 64), (300, 520, 511), (17, 129, 257), (1000, 700, 300)])
@pytest.mark.parametrize("B", [17, 33, 130, 257])
def test_prefill_parity_small(m, n, r, B):
    L = synth.make_layer(m, n, r, B, cfg=5, layer=m + n + r + B)
    layer = G.pack_layer(L)
    ref = G.oracle(L, "dense")
    y32 = G.run(L, layer, y_dtype=torch.float32)
    ybf = G.run(L, layer, y_dtype=torch.bfloat16)
    assert G.rel_l2(y32, ref) <= TOL32
    G.check_bf16_output(ybf, ref, y32)


@pytest.mark.parametrize("B", [1, 3, 16])
def test_gemm_path_small_batch(B):
    """The GEMM kernels at small B, forced, against the oracle."""
    L = synth.make_layer(300, 520, 511, B, cfg=5)
    ref = G.oracle(L, "dense")
    y = G.run(L, y_dtype=torch.float32, path="gemm")
    assert G.rel_l2(y, ref) <= TOL32


def test_prefill_exact_integers():
    """x in {-3..3}, s1, s2, g in {1, 2}, n = 64: every fp16 operand is a small
    integer (|T'| <= 2 * 6 * 64 = 768 < 2^11), so the fp32 result is exact."""
    m, n, r, B = 300, 64, 96, 40
    rng = np.random.default_rng(7)
    L = synth.make_integer_layer(m, n, r, B, seed=3)
    L.g = rng.choice([1.0, 2.0], size=r).astype(np.float32)
    ref = G.oracle(L, "factored")
    y = G.run(L, y_dtype=torch.float32)
    assert np.array_equal(y, ref)


def test_prefill_ksplit_exact_integers():
    """A small-rank shape (6 output tiles, 34 K steps) whose first GEMM runs in
    7 K ranges (5 steps each, the last 4), the partials summed by the mid
    kernel.  x is zero except 48 columns spread over all ranges, so every
    partial and every fp16 operand is a small integer or half-integer and the
    fp32 result is exact."""
    m, n, r, B = 200, 2100, 150, 300
    L = synth.make_integer_layer(m, n, r, B, seed=11)
    keep = np.linspace(0, n - 1, 48).astype(int)
    mask = np.zeros(n, bool)
    mask[keep] = True
    L.x[:, ~mask] = 0.0
    layer = G.pack_layer(L)
    # the workspace beyond the two fp16 operand copies holds the fp32 T: more
    # than one B x r partial of it means the K split is taken
    f16_copies = B * (-(-n // 128) * 128 + -(-r // 128) * 128) * 2
    assert nq.workspace_bytes(layer, B, "gemm") - f16_copies >= 2 * B * r * 4
    ref = G.oracle(L, "factored")
    y = G.run(L, layer, y_dtype=torch.float32)
    assert np.array_equal(y, ref)


def test_prefill_ksplit_parity():
    """The same split shape with random fp16 scales and inputs, fp32 and bf16
    outputs, against the fp64 oracle."""
    L = synth.make_layer(200, 2100, 150, 300, cfg=5, layer=4)
    layer = G.pack_layer(L)
    ref = G.oracle(L, "dense")
    y32 = G.run(L, layer, y_dtype=torch.float32)
    ybf = G.run(L, layer, y_dtype=torch.bfloat16)
    assert G.rel_l2(y32, ref) <= TOL32
    G.check_bf16_output(ybf, ref, y32)


@pytest.mark.parametrize("x_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("scale_dtype", ["f32", "f16"])
@pytest.mark.parametrize("n,r", [(1024, 200), (1030, 201)])
def test_prefill_dtypes(x_dtype, scale_dtype, n, r):
    """Every activation / scale dtype pair on the prefill path, with column
    counts that are (n = 1024, r = 200) and are not (1030, 201) multiples of
    four, so the row kernels run both their four-column and one-column forms;
    both shapes also take the K split (2 output tiles; 16 and 18 K steps in 4
    ranges, the last of the second one shorter)."""
    L = synth.make_layer(150, n, r, 40, cfg=5, layer=n + r, x_dtype=x_dtype, scale_dtype=scale_dtype)
    ref = G.oracle(L, "dense")
    y = G.run(L, y_dtype=torch.float32)
    assert G.rel_l2(y, ref) <= TOL32


def test_prefill_batch_rows_independent():
    L = synth.make_layer(500, 400, 200, 64, cfg=6)
    layer = G.pack_layer(L)
    y = G.run(L, layer, y_dtype=torch.float32)
    for b in (0, 17, 63):
        yb = G.run(L, layer, y_dtype=torch.float32, path="gemm", x_override=L.x[b:b + 1])
        assert np.array_equal(yb[0], y[b])  # same row, same kernels: identical


@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
def test_config5_llama70b_prefill_sampled(name):
    """2048 tokens through one layer of each distinct 70B shape at 0.8 bpw, in
    the launch configuration of the prefill benchmark; 24 sampled tokens are
    checked against the factored fp64 oracle over all m outputs."""
    m, n = synth.LLAMA70B[name]
    r = O.rank_for_bits(m, n, 0.8, 16)
    B = 2048
    L = synth.make_layer(m, n, r, B, cfg=5, block=0, layer=synth.LAYER_ORDER.index(name))
    layer = G.pack_layer(L)
    y = G.run(L, layer, y_dtype=torch.bfloat16)
    rows = np.random.default_rng(5).choice(B, 24, replace=False)
    ref = O.linear_factored(L.x[rows].astype(np.float64), L.U, L.V, L.s1.astype(np.float64),
                            L.g.astype(np.float64), L.s2.astype(np.float64))
    rr = G.bf16_round(ref)
    assert G.rel_l2(y[rows], ref) <= G.TOL + G.rel_l2(rr, ref), G.rel_l2(y[rows], ref)
