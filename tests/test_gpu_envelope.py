"""GPU: the rank-l envelope (MDBF) forward, nq_linear_fwd_envelope, against
the fp64 envelope oracle; at one term it is the plain decode path bit for bit."""
import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
import synth
from oracle import nq_oracle as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _env_case(m, n, r, B, env, cfg, x_dtype="bf16", scale_dtype="f16"):
    L = synth.make_layer(m, n, r, B, cfg=cfg, layer=env, x_dtype=x_dtype, scale_dtype=scale_dtype)
    rng = np.random.default_rng([cfg, m, n, r, env])
    sd = {"f16": np.float16, "f32": np.float32}[scale_dtype]
    S1 = np.stack([L.s1] + [synth.scales(rng, m, sd) for _ in range(env - 1)])
    S2 = np.stack([L.s2] + [synth.scales(rng, n, sd) for _ in range(env - 1)])
    return L, S1, S2


def _run(L, layer, S1, S2, y_dtype):
    x = G.x_tensor(L.x, L.x_dtype)
    y = nq.linear_envelope(x, layer, G.to_torch_scale(S1), G.to_torch_scale(S2), out_dtype=y_dtype)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _ref(L, S1, S2):
    return O.linear_envelope_dense(L.x.astype(np.float64), L.U, L.V, S1.astype(np.float64), L.g.astype(np.float64),
                                   S2.astype(np.float64))


SHAPES = [(256, 256, 64), (63, 17, 5), (100, 300, 130), (17, 129, 257), (300, 520, 511), (1024, 1100, 600)]
ENV_B = [(2, 1), (2, 2), (3, 1), (4, 1)]


@pytest.mark.parametrize("m,n,r", SHAPES)
@pytest.mark.parametrize("env,B", ENV_B)
def test_envelope_parity(m, n, r, env, B):
    L, S1, S2 = _env_case(m, n, r, B, env, cfg=60)
    layer = G.pack_layer(L)
    ref = _ref(L, S1, S2)
    y32 = _run(L, layer, S1, S2, torch.float32)
    ybf = _run(L, layer, S1, S2, torch.bfloat16)
    assert G.rel_l2(y32, ref) <= 3e-4
    G.check_bf16_output(ybf, ref, y32)


def test_envelope_fp32_scales_and_inputs():
    L, S1, S2 = _env_case(200, 300, 100, 1, 3, cfg=61, x_dtype="f32", scale_dtype="f32")
    y = _run(L, G.pack_layer(L), S1, S2, torch.float32)
    assert G.rel_l2(y, _ref(L, S1, S2)) <= 3e-4


@pytest.mark.parametrize("B", [1, 2, 4])
def test_single_term_equals_decode_path_bit_for_bit(B):
    """4096 outputs: tall enough that the plain decode path also uses the
    row-split stage 2 the envelope runs on, so the two plans coincide."""
    L, S1, S2 = _env_case(4096, 1100, 600, B, 1, cfg=62)
    layer = G.pack_layer(L)
    assert np.array_equal(_run(L, layer, S1, S2, torch.float32), G.run(L, layer, y_dtype=torch.float32,
                                                                        path="decode"))


def test_envelope_exact_integers():
    """Integer x, scales in {1, 2}, g in {1, 1/2}: every term is exact, so is the sum."""
    L = synth.make_integer_layer(96, 200, 40, 1, seed=63)
    rng = np.random.default_rng(63)
    S1 = np.stack([L.s1, rng.choice([1.0, 2.0], size=96).astype(L.s1.dtype)])
    S2 = np.stack([L.s2, rng.choice([1.0, 2.0], size=200).astype(L.s2.dtype)])
    y = _run(L, G.pack_layer(L), S1, S2, torch.float32)
    assert np.array_equal(y, O.linear_envelope_factored(L.x.astype(np.float64), L.U, L.V, S1.astype(np.float64),
                                                        L.g.astype(np.float64), S2.astype(np.float64)))


def test_envelope_llama70b_gate_two_terms():
    m, n = synth.LLAMA70B["gate"]
    r = nq.rank_for_bits(m, n, 0.8, 16)
    L, S1, S2 = _env_case(m, n, r, 1, 2, cfg=4)
    layer = G.pack_layer(L)
    ref = O.linear_envelope_factored(L.x.astype(np.float64), L.U, L.V, S1.astype(np.float64),
                                     L.g.astype(np.float64), S2.astype(np.float64))
    y32 = _run(L, layer, S1, S2, torch.float32)
    assert G.rel_l2(y32, ref) <= 3e-4
    G.check_bf16_output(_run(L, layer, S1, S2, torch.bfloat16), ref, y32)


def test_envelope_beyond_four_rows_is_unsupported():
    L, S1, S2 = _env_case(64, 96, 16, 3, 2, cfg=64)
    with pytest.raises(nq.NQError) as e:
        _run(L, G.pack_layer(L), S1, S2, torch.float32)
    assert e.value.status == nq.NQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("env,B", [(3, 1), (4, 1), (2, 2)])
def test_envelope_parity_70b_rank(env, B):
    """Rank 5079 (the 70B gate/up/down rank at 0.8 bpw): three and four terms
    need the plans that use more than 64 KiB of LDS per workgroup."""
    m, n, r = 2048, 8192, 5079
    L, S1, S2 = _env_case(m, n, r, B, env, cfg=61)
    layer = G.pack_layer(L)
    ref = O.linear_envelope_factored(L.x.astype(np.float64), L.U, L.V, S1.astype(np.float64),
                                     L.g.astype(np.float64), S2.astype(np.float64))
    print(f"envelope 70b rank env={env} B={B}", flush=True)
    y32 = _run(L, layer, S1, S2, torch.float32)
    ybf = _run(L, layer, S1, S2, torch.bfloat16)
    assert G.rel_l2(y32, ref) <= 3e-4
    G.check_bf16_output(ybf, ref, y32)
