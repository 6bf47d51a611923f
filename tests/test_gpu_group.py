"""GPU: layer groups (q/k/v and gate/up share x) through nq_linear_fwd_group:
every output against the fp64 oracle of its own layer, bit equality with the
single-layer decode path where the plans coincide, and large batches as
passes of four rows."""
import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _group(shapes, n, B, cfg, x_dtype="bf16", scale_dtype="f16"):
    Ls = [synth.make_layer(m, n, r, B, cfg=cfg, layer=i, x_dtype=x_dtype, scale_dtype=scale_dtype)
          for i, (m, r) in enumerate(shapes)]
    x = Ls[0].x  # one input for the whole group
    for L in Ls:
        L.x = x
    return Ls, [G.pack_layer(L) for L in Ls]


def _run_group(Ls, layers, y_dtype):
    x = G.x_tensor(Ls[0].x, Ls[0].x_dtype)
    ys = nq.linear_group(x, layers, out_dtype=y_dtype)
    torch.cuda.synchronize()
    return [y.float().cpu().numpy().astype(np.float64) for y in ys]


GROUPS = [
    ("qkv-like", [(300, 129), (64, 40), (64, 40)], 520),
    ("gate-up-like", [(700, 300), (700, 300)], 256),
    ("ragged", [(17, 257), (1, 1), (100, 130)], 129),
    ("four", [(128, 64), (256, 100), (48, 17), (512, 511)], 1000),
]


@pytest.mark.parametrize("name,shapes,n", GROUPS)
@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_group_parity_small(name, shapes, n, B):
    Ls, layers = _group(shapes, n, B, cfg=30 + B)
    y32 = _run_group(Ls, layers, torch.float32)
    ybf = _run_group(Ls, layers, torch.bfloat16)
    for L, a, b in zip(Ls, y32, ybf):
        ref = G.oracle(L, "dense")
        assert G.rel_l2(a, ref) <= 3e-4, (name, L.m, L.r)
        G.check_bf16_output(b, ref, a)


def test_group_fp32_inputs_and_scales():
    Ls, layers = _group([(200, 64), (96, 50)], 300, 2, cfg=37, x_dtype="f32", scale_dtype="f32")
    for L, y in zip(Ls, _run_group(Ls, layers, torch.float32)):
        assert G.rel_l2(y, G.oracle(L, "dense")) <= 3e-4


def test_single_layer_group_equals_decode_path_bit_for_bit():
    """A group of one is planned exactly like the single-layer decode path."""
    for (m, n, r, B) in [(1000, 1100, 600, 1), (300, 520, 129, 4), (1024, 8192, 710, 1)]:
        Ls, layers = _group([(m, r)], n, B, cfg=38)
        yg = _run_group(Ls, layers, torch.float32)[0]
        yd = G.run(Ls[0], layers[0], y_dtype=torch.float32, path="decode")
        assert np.array_equal(yg, yd)


@pytest.mark.parametrize("B,shapes,n", [(5, [(300, 129), (64, 40)], 520), (17, [(300, 129), (64, 40)], 520),
                                         (6, [(17, 257), (1, 1), (100, 130)], 129)])
def test_group_beyond_fused_batch_runs_in_passes(B, shapes, n):
    """B > 4 runs as passes of four rows (and one of B mod 4) through the fused
    group path: every output against the oracle, and every pass equal bit for
    bit to the group call on its rows alone (n = 129: later passes start at
    rows that are not 16-byte aligned)."""
    Ls, layers = _group(shapes, n, B, cfg=39)
    yg = _run_group(Ls, layers, torch.float32)
    for L, y in zip(Ls, yg):
        assert G.rel_l2(y, G.oracle(L, "factored")) <= 3e-4
    x_all = Ls[0].x
    for b0 in range(0, B, 4):
        for L in Ls:
            L.x = x_all[b0:b0 + 4]
        part = _run_group(Ls, layers, torch.float32)
        for y, yp in zip(yg, part):
            assert np.array_equal(y[b0:b0 + 4], yp)


def test_group_deterministic():
    Ls, layers = _group([(300, 129), (64, 40), (64, 40)], 520, 1, cfg=40)
    a = _run_group(Ls, layers, torch.bfloat16)
    b = _run_group(Ls, layers, torch.bfloat16)
    assert all(np.array_equal(u, v) for u, v in zip(a, b))


@pytest.mark.parametrize("which", ["qkv", "gate_up"])
@pytest.mark.parametrize("B", [1, 4])
def test_config4_llama70b_groups(which, B):
    """The 70B block's shared-input groups at 0.8 bpw, B = 1 and 4 (at B = 4
    the plan needs more than 64 KiB of LDS per workgroup), each output against
    the factored fp64 oracle of its layer."""
    names = ["q", "k", "v"] if which == "qkv" else ["gate", "up"]
    Ls = []
    for i, nm in enumerate(names):
        m, n = synth.LLAMA70B[nm]
        r = nq.rank_for_bits(m, n, 0.8, 16)
        Ls.append(synth.make_layer(m, n, r, B, cfg=4, block=0, layer=synth.LAYER_ORDER.index(nm)))
    for L in Ls[1:]:
        L.x = Ls[0].x
    layers = [G.pack_layer(L) for L in Ls]
    ybf = _run_group(Ls, layers, torch.bfloat16)
    y32 = _run_group(Ls, layers, torch.float32)
    for L, a, b in zip(Ls, y32, ybf):
        ref = G.oracle(L, "factored")
        assert G.rel_l2(a, ref) <= 3e-4
        G.check_bf16_output(b, ref, a)
