"""GPU parity of the packed layout and the batch-1..16 forward against the fp64
oracle.  Every call goes through the C ABI of libnq.so."""
import numpy as np
import pytest
import scipy.linalg
import torch

import binary_rank_gemv_packed_amd as nq
import synth
from oracle import nq_oracle as O
from tests import gpu_util as G
from tests.layout_decoder import decode_blob

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ pack / unpack
@pytest.mark.parametrize("m,n,r", [(1, 1, 1), (63, 17, 5), (256, 256, 64), (100, 300, 130),
                                   (1024, 8192, 710), (11008, 4096, 2369)])
def test_pack_unpack_roundtrip_bit_exact(m, n, r):
    L = synth.make_layer(m, n, r, 1, cfg=90, layer=m % 97)
    layer = G.pack_layer(L)
    U, V = nq.unpack(layer)
    assert np.array_equal(U.cpu().numpy(), L.U)
    assert np.array_equal(V.cpu().numpy(), L.V)


@pytest.mark.parametrize("m,n,r,sdt", [(63, 17, 5, "f16"), (256, 256, 64, "f32"), (40, 200, 129, "f16")])
def test_blob_matches_documented_layout(m, n, r, sdt):
    L = synth.make_layer(m, n, r, 1, cfg=91, scale_dtype=sdt)
    layer = G.pack_layer(L)
    blob = layer.blob.cpu().numpy().tobytes()
    h, U, V, s1, g, s2 = decode_blob(blob)
    assert (h["magic"], h["version"], h["m"], h["n"], h["r"], h["bad"]) == (0x3142514E, 1, m, n, r, 0)
    assert h["total"] == len(blob)
    assert np.array_equal(U, L.U) and np.array_equal(V, L.V)
    assert np.array_equal(s1, L.s1) and np.array_equal(g, L.g) and np.array_equal(s2, L.s2)


@pytest.mark.parametrize("bad_value", [0, 2, -128])
@pytest.mark.parametrize("which", ["U", "V"])
def test_pack_rejects_entries_other_than_pm1(bad_value, which):
    L = synth.make_layer(33, 70, 9, 1, cfg=92)
    M = getattr(L, which)
    M[M.shape[0] // 2, 3] = bad_value
    with pytest.raises(nq.NQError) as e:
        G.pack_layer(L)
    assert e.value.status == nq.NQ_ERR_NOT_PM1


# ------------------------------------------------------------------ parity, small shapes
SMALL = [(256, 256, 64), (63, 17, 5), (100, 300, 130), (1, 1, 1), (16, 128, 128), (17, 129, 257),
         (300, 520, 511)]


PATH_B = [("decode", B) for B in (1, 2, 3, 4, 5, 8, 13, 16)] + [("gemv", B) for B in (1, 2, 3, 4, 5, 8, 13, 16)]


@pytest.mark.parametrize("m,n,r", SMALL)
@pytest.mark.parametrize("path,B", PATH_B)
def test_gemv_parity_small(m, n, r, path, B):
    L = synth.make_layer(m, n, r, B, cfg=1, layer=m + n + r)
    layer = G.pack_layer(L)
    ref = G.oracle(L, "dense")
    y32 = G.run(L, layer, y_dtype=torch.float32, path=path)
    ybf = G.run(L, layer, y_dtype=torch.bfloat16, path=path)
    e32 = G.rel_l2(y32, ref)
    assert e32 <= 3e-4, (e32, B)
    G.check_bf16_output(ybf, ref, y32)


def test_config1_fp32():
    """256 x 256, r = 64, B = 1, fp32 x and scales, |N(0,1)|+0.1 scales."""
    L = synth.make_layer(256, 256, 64, 1, cfg=1, scale_dtype="f32", x_dtype="f32")
    ref = G.oracle(L, "dense")
    y = G.run(L, y_dtype=torch.float32)
    assert G.rel_l2(y, ref) <= 1e-5


def test_empty_batch_is_no_op():
    L = synth.make_layer(64, 64, 16, 1)
    layer = G.pack_layer(L)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=G.DEV)
    y = nq.linear(x, layer)
    assert y.shape == (0, 64)


# ------------------------------------------------------------------ exactness and invariants
@pytest.mark.parametrize("m,n,r", [(256, 256, 64), (1024, 8192, 710), (300, 520, 511), (4096, 4096, 1619)])
@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("path", ["decode", "gemv"])
def test_exact_integer_inputs_bit_exact(m, n, r, B, path):
    """x in {-3..3}, s1, s2 in {1, 2}, g in {1, 1/2}: every partial sum is an exact
    small dyadic rational, so the fp32 result equals the oracle exactly.  The
    activation pieces hold 16 significant bits per 32-value block, so the exact
    intermediate t' = g * V^T (s2 x) must stay below 2^15 in magnitude."""
    L = synth.make_integer_layer(m, n, r, B, seed=m + r)
    t = (L.x.astype(np.float64) * L.s2.astype(np.float64)) @ L.V.astype(np.float64) * L.g.astype(np.float64)
    assert np.max(np.abs(t)) < 2 ** 15 and np.max(np.abs(L.x * L.s2)) < 2 ** 15
    ref = G.oracle(L, "factored")
    y = G.run(L, y_dtype=torch.float32, path=path)
    assert np.array_equal(y, ref)


@pytest.mark.parametrize("p", [4, 7, 8])
def test_hadamard_identity_exact(p):
    """U = V = H_n, s1 = s2 = 1, g = 1/n: W_hat = I, so y == x exactly."""
    n = 2 ** p
    H = scipy.linalg.hadamard(n).astype(np.int8)
    rng = np.random.default_rng(p)
    x = rng.integers(-9, 10, size=(2, n)).astype(np.float32)
    L = synth.Layer(n, n, n, H, H.copy(), np.ones(n, np.float32), np.full(n, 1.0 / n, np.float32),
                    np.ones(n, np.float32), x, "f32", "f32")
    y = G.run(L, y_dtype=torch.float32)
    assert np.array_equal(y, x.astype(np.float64))


def test_sign_flip_invariance_exact():
    L = synth.make_integer_layer(96, 200, 40, 2, seed=5)
    y0 = G.run(L, y_dtype=torch.float32)
    for k in (0, 17, 39):
        L.U[:, k] *= -1
        L.V[:, k] *= -1
        assert np.array_equal(G.run(L, y_dtype=torch.float32), y0)


def test_batch_rows_independent():
    L = synth.make_layer(700, 900, 300, 7, cfg=3)
    layer = G.pack_layer(L)
    y = G.run(L, layer, y_dtype=torch.float32)
    for b in range(7):
        yb = G.run(L, layer, y_dtype=torch.float32, x_override=L.x[b:b + 1])
        assert G.rel_l2(yb[0], y[b]) <= 3e-4


@pytest.mark.parametrize("path", ["decode", "gemv"])
def test_deterministic_reruns(path):
    L = synth.make_layer(2000, 3000, 800, 2, cfg=4)
    layer = G.pack_layer(L)
    a = G.run(L, layer, y_dtype=torch.float32, path=path)
    b = G.run(L, layer, y_dtype=torch.float32, path=path)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("m,n,r", [(256, 256, 64), (300, 520, 511), (4096, 4096, 1619)])
def test_valu_path_parity(m, n, r):
    L = synth.make_layer(m, n, r, 1, cfg=5)
    ref = G.oracle(L, "factored")
    y = G.run(L, y_dtype=torch.float32, path="valu")
    assert G.rel_l2(y, ref) <= 1e-5


# ------------------------------------------------------------------ Llama-shaped layers
def _cfg_layers(shapes, bpw):
    out = []
    for name in synth.LAYER_ORDER:
        m, n = shapes[name]
        if (m, n) not in [(a, b) for _, (a, b) in out]:
            out.append((name, (m, n)))
    return [(name, m, n, O.rank_for_bits(m, n, bpw, 16)) for name, (m, n) in out]


@pytest.mark.parametrize("name,m,n,r", _cfg_layers(synth.LLAMA7B, 1.0))
def test_config2_llama7b_1bpw(name, m, n, r):
    L = synth.make_layer(m, n, r, 1, cfg=2, layer=synth.LAYER_ORDER.index(name))
    ref = G.oracle(L, "factored")
    assert G.rel_l2(G.run(L), ref) <= G.TOL


@pytest.mark.parametrize("bpw", [0.55, 0.8])
@pytest.mark.parametrize("name,m,n", [("q", 4096, 4096), ("gate", 11008, 4096), ("down", 4096, 11008)])
def test_config3_llama7b_batch_sweep(bpw, name, m, n):
    r = O.rank_for_bits(m, n, bpw, 16)
    L16 = synth.make_layer(m, n, r, 16, cfg=3, layer=synth.LAYER_ORDER.index(name))
    layer = G.pack_layer(L16)
    for B in (1, 2, 4, 8, 16):
        x = L16.x[:B]
        ref = G.oracle(L16, "factored", x=x)
        for path in (["auto", "gemv"] if B <= 4 else ["auto"]):
            y = G.run(L16, layer, x_override=x, path=path)
            assert G.rel_l2(y, ref) <= G.TOL, (B, path, G.rel_l2(y, ref))


@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
def test_config4_llama70b_layer(name):
    """One layer of each distinct 70B shape at 0.8 bpw, B = 1, full output against
    the factored fp64 oracle (same launch configuration as the decode benchmark)."""
    m, n = synth.LLAMA70B[name]
    r = O.rank_for_bits(m, n, 0.8, 16)
    L = synth.make_layer(m, n, r, 1, cfg=4, block=0, layer=synth.LAYER_ORDER.index(name))
    ref = G.oracle(L, "factored")
    assert G.rel_l2(G.run(L), ref) <= G.TOL


@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
def test_config4_llama70b_batched(name):
    """70B shapes at 0.8 bpw with B = 3, 4 and 16 on the decode path (one pass
    over the weights per four batch rows: at these ranks the t' image of three
    or four rows needs more than 64 KiB of LDS), every output against the
    factored fp64 oracle, fp32 and bf16 outputs."""
    m, n = synth.LLAMA70B[name]
    r = O.rank_for_bits(m, n, 0.8, 16)
    L16 = synth.make_layer(m, n, r, 16, cfg=4, block=1, layer=synth.LAYER_ORDER.index(name))
    layer = G.pack_layer(L16)
    for B in (3, 4, 16):
        x = L16.x[:B]
        ref = G.oracle(L16, "factored", x=x)
        print(f"70b batched {name} B={B}", flush=True)
        y32 = G.run(L16, layer, x_override=x, y_dtype=torch.float32, path="decode")
        assert G.rel_l2(y32, ref) <= 3e-4, (B, G.rel_l2(y32, ref))
        y = G.run(L16, layer, x_override=x, path="decode")
        assert G.rel_l2(y, ref) <= G.TOL, (B, G.rel_l2(y, ref))
