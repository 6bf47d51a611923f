"""Edge cases of the forward through the C ABI: guard bytes around the output
and the workspace, zero and non-finite activations, activations spanning a
huge dynamic range, and the batch-size limits of each path."""
import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SENT = 0x5A


@pytest.mark.parametrize("path,B", [("decode", 1), ("decode", 4), ("gemv", 3), ("gemv", 16)])
@pytest.mark.parametrize("m,n,r", [(63, 200, 129), (1000, 700, 300)])
def test_guard_bytes_untouched(path, B, m, n, r):
    """Writes stay inside y[B, m] and inside nq_workspace_bytes of workspace."""
    L = synth.make_layer(m, n, r, B, cfg=7)
    layer = G.pack_layer(L)
    pad = 4096
    ybuf = torch.full((B * m * 4 + 2 * pad,), SENT, dtype=torch.uint8, device=G.DEV)
    y = ybuf[pad:pad + B * m * 4].view(torch.float32).view(B, m)
    wsb = nq.workspace_bytes(layer, B)
    wbuf = torch.full((wsb + pad,), SENT, dtype=torch.uint8, device=G.DEV)
    x = G.x_tensor(L.x, L.x_dtype)
    nq.linear_into(x, layer, y, wbuf, path=path)
    torch.cuda.synchronize()
    yb = ybuf.cpu().numpy()
    assert np.all(yb[:pad] == SENT) and np.all(yb[-pad:] == SENT)
    assert np.all(wbuf[wsb:].cpu().numpy() == SENT)
    ref = G.oracle(L, "factored")
    assert G.rel_l2(y.cpu().numpy(), ref) <= 3e-4


@pytest.mark.parametrize("path,B", [("decode", 1), ("decode", 2), ("gemv", 8)])
def test_zero_input_gives_exact_zero(path, B):
    L = synth.make_layer(300, 520, 200, B, cfg=8)
    y = G.run(L, y_dtype=torch.float32, path=path, x_override=np.zeros_like(L.x))
    assert np.array_equal(y, np.zeros_like(y))


@pytest.mark.parametrize("path", ["decode", "gemv"])
@pytest.mark.parametrize("bad", [np.nan, np.inf])
def test_non_finite_input_propagates(path, bad):
    """A NaN or an infinite activation makes every output non-finite, as in the
    oracle (every weight is non-zero)."""
    L = synth.make_layer(200, 300, 64, 2, cfg=9, x_dtype="f32")
    x = L.x.copy()
    x[1, 17] = bad
    y = G.run(L, y_dtype=torch.float32, path=path, x_override=x)
    ref = G.oracle(L, "factored", x=x)
    assert np.all(np.isfinite(y[0])) and np.all(np.isfinite(ref[0]))
    assert not np.any(np.isfinite(y[1])) and not np.any(np.isfinite(ref[1]))


@pytest.mark.parametrize("path", ["decode", "gemv"])
def test_huge_dynamic_range(path):
    """Activations from 1e-30 to 1e30 (fp32 x): each 32-value block gets its own
    scale, so the relative L2 error stays at the usual level."""
    rng = np.random.default_rng(11)
    L = synth.make_layer(256, 512, 96, 2, cfg=10, x_dtype="f32")
    x = (rng.standard_normal((2, 512)) * 10.0 ** rng.uniform(-30, 30, size=(2, 512))).astype(np.float32)
    y = G.run(L, y_dtype=torch.float32, path=path, x_override=x)
    ref = G.oracle(L, "factored", x=x)
    assert G.rel_l2(y, ref) <= 3e-4


def test_path_batch_limits():
    L = synth.make_layer(64, 64, 16, 17)
    layer = G.pack_layer(L)
    x = G.x_tensor(L.x, L.x_dtype)
    with pytest.raises(nq.NQError) as e:
        nq.linear(x, layer, path="decode")  # 17 rows: beyond the chunked decode path
    assert e.value.status == nq.NQ_ERR_UNSUPPORTED
    with pytest.raises(nq.NQError) as e:
        nq.linear(x, layer, path="gemv")
    assert e.value.status == nq.NQ_ERR_UNSUPPORTED
