"""GPU: the transposed product through the transposing pack.  The layer
nq_transpose_layer writes must be the very blob that packing the swapped
factors gives, and every forward path on it must match the oracle's
dx = dy W_hat (and be adjoint to the forward)."""
import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
import synth
from oracle import nq_oracle as O
from tests import gpu_util as G
from tests.layout_decoder import decode_blob

pytestmark = pytest.mark.gpu

SHAPES = [(63, 17, 5), (256, 256, 64), (100, 300, 130), (1, 1, 1), (17, 129, 257), (300, 520, 511),
          (1024, 8192, 710)]


def _regions(layer):
    blob = layer.blob.cpu().numpy().tobytes()
    h = decode_blob(blob)[0]
    return blob, h


@pytest.mark.parametrize("m,n,r", SHAPES)
@pytest.mark.parametrize("sdt", ["f16", "f32"])
def test_transposed_blob_equals_packing_swapped_factors(m, n, r, sdt):
    L = synth.make_layer(m, n, r, 1, cfg=50, layer=m + r, scale_dtype=sdt)
    layer = G.pack_layer(L)
    tl = nq.transpose(layer)
    direct = nq.pack(torch.from_numpy(L.V).to(G.DEV), torch.from_numpy(L.U).to(G.DEV), G.to_torch_scale(L.s2),
                     G.to_torch_scale(L.g), G.to_torch_scale(L.s1))
    a, ha = _regions(tl)
    b, hb = _regions(direct)
    assert ha == hb
    assert a[:80] == b[:80]  # the header as stored
    for lo, hi in [(ha["off_u"], ha["off_vt"]), (ha["off_vt"], ha["off_s1"])]:
        assert a[lo:hi] == b[lo:hi]  # packed words, padding bits included
    _, U2, V2, s1, g, s2 = decode_blob(a)
    assert np.array_equal(U2, L.V) and np.array_equal(V2, L.U)
    assert np.array_equal(s1, L.s2) and np.array_equal(g, L.g) and np.array_equal(s2, L.s1)


def test_double_transpose_restores_the_layer():
    L = synth.make_layer(300, 520, 511, 1, cfg=51)
    layer = G.pack_layer(L)
    back = nq.transpose(nq.transpose(layer))
    a, ha = _regions(back)
    b, hb = _regions(layer)
    assert ha == hb
    for lo, hi in [(ha["off_u"], ha["off_vt"]), (ha["off_vt"], ha["off_s1"])]:
        assert a[lo:hi] == b[lo:hi]


PATH_B = [("decode", 1), ("decode", 3), ("gemv", 5), ("gemv", 16), ("gemm", 40)]


@pytest.mark.parametrize("m,n,r", SHAPES)
@pytest.mark.parametrize("path,B", PATH_B)
def test_transposed_product_parity(m, n, r, path, B):
    L = synth.make_layer(m, n, r, B, cfg=52, layer=n + r)
    layer = G.pack_layer(L)
    tl = nq.transpose(layer)
    dy = synth.activations(np.random.default_rng([52, m, n, r, B]), B, m, "bf16")
    ref = O.linear_transposed_dense(dy.astype(np.float64), L.U, L.V, L.s1.astype(np.float64),
                                    L.g.astype(np.float64), L.s2.astype(np.float64))
    dyt = G.x_tensor(dy, "bf16")
    dx32 = nq.linear(dyt, tl, out_dtype=torch.float32, path=path).cpu().numpy().astype(np.float64)
    dxbf = nq.linear(dyt, tl, out_dtype=torch.bfloat16, path=path).float().cpu().numpy().astype(np.float64)
    assert G.rel_l2(dx32, ref) <= (1e-3 if path == "gemm" else 3e-4)
    if path != "gemm":
        G.check_bf16_output(dxbf, ref, dx32)
    else:
        assert G.rel_l2(dxbf, ref) <= G.TOL + G.rel_l2(G.bf16_round(ref), ref)


def test_adjointness_on_the_gpu():
    """<W x, dy> = <x, W^T dy> for the GPU's own forward and transposed outputs."""
    L = synth.make_layer(700, 900, 300, 4, cfg=53)
    layer = G.pack_layer(L)
    tl = nq.transpose(layer)
    rng = np.random.default_rng(53)
    dy = synth.activations(rng, 4, 700, "bf16")
    y = G.run(L, layer, y_dtype=torch.float32)
    dx = nq.linear(G.x_tensor(dy, "bf16"), tl, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    lhs = np.sum(y * dy, axis=1)
    rhs = np.sum(L.x.astype(np.float64) * dx, axis=1)
    scale = np.linalg.norm(y, axis=1) * np.linalg.norm(dy, axis=1)
    assert np.all(np.abs(lhs - rhs) <= 1e-4 * scale)


@pytest.mark.parametrize("name", ["gate", "down", "k"])
def test_config4_llama70b_transposed(name):
    m, n = synth.LLAMA70B[name]
    r = nq.rank_for_bits(m, n, 0.8, 16)
    L = synth.make_layer(m, n, r, 1, cfg=4, block=0, layer=synth.LAYER_ORDER.index(name))
    tl = nq.transpose(G.pack_layer(L))
    dy = synth.activations(np.random.default_rng([4, 54, m]), 1, m, "bf16")
    ref = O.linear_transposed_factored(dy.astype(np.float64), L.U, L.V, L.s1.astype(np.float64),
                                       L.g.astype(np.float64), L.s2.astype(np.float64))
    dyt = G.x_tensor(dy, "bf16")
    dx32 = nq.linear(dyt, tl, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    dxbf = nq.linear(dyt, tl, out_dtype=torch.bfloat16).float().cpu().numpy().astype(np.float64)
    assert G.rel_l2(dx32, ref) <= 3e-4
    G.check_bf16_output(dxbf, ref, dx32)
