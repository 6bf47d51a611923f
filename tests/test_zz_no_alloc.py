"""GPU: the entry point that allocates nothing (nq_linear_fwd_noalloc) against the
workspace entry point (nq_linear_fwd) through the C ABI: identical outputs on
two calls in a row, the second with a smaller input."""
import ctypes

import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
import synth
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _both(L, layer, ydt):
    x = G.x_tensor(L.x, L.x_dtype)
    B = x.shape[0]
    y_ws = torch.empty((B, layer.m), dtype=ydt, device=G.DEV)
    ws = nq.new_workspace(layer, B)
    st = torch.cuda.current_stream().cuda_stream
    lib = nq.lib()
    assert lib.nq_linear_fwd(layer.ref, x.data_ptr(), nq._DT[x.dtype], y_ws.data_ptr(), nq._DT[ydt], B,
                             ws.data_ptr(), ws.numel(), st) == nq.NQ_OK
    y_na = torch.full((B, layer.m), float("nan"), dtype=ydt, device=G.DEV)
    assert lib.nq_linear_fwd_noalloc(layer.ref, x.data_ptr(), nq._DT[x.dtype], y_na.data_ptr(), nq._DT[ydt], B,
                                     st) == nq.NQ_OK, lib.nq_last_error()
    torch.cuda.synchronize()
    return y_ws.float().cpu().numpy(), y_na.float().cpu().numpy()


@pytest.mark.parametrize("ydt", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry_point_twice(ydt):
    # first call: decode path at B = 4 on a larger layer; second: smaller layer, B = 1
    for (m, n, r, B) in [(1000, 1100, 600, 4), (300, 520, 129, 1)]:
        L = synth.make_layer(m, n, r, B, cfg=11, layer=m)
        layer = G.pack_layer(L)
        y_ws, y_na = _both(L, layer, ydt)
        assert np.array_equal(y_ws, y_na)
        ref = G.oracle(L, "factored")
        bar = 1e-3 if ydt == torch.float32 else G.TOL + G.rel_l2(G.bf16_round(ref), ref)
        assert G.rel_l2(y_na, ref) <= bar


def test_noalloc_other_paths_twice():
    # gemv path (B = 9) then prefill path (B = 40), each against the workspace entry point
    for (m, n, r, B) in [(700, 900, 300, 9), (200, 300, 64, 40)]:
        L = synth.make_layer(m, n, r, B, cfg=12, layer=n)
        layer = G.pack_layer(L)
        y_ws, y_na = _both(L, layer, torch.float32)
        assert np.array_equal(y_ws, y_na)


def test_noalloc_rejects_oversize():
    lay = nq.empty_layer(8192, 28672, 5079)
    x = torch.zeros((2048, 28672), dtype=torch.bfloat16, device=G.DEV)
    y = torch.empty((2048, 8192), dtype=torch.bfloat16, device=G.DEV)
    with pytest.raises(nq.NQError) as e:
        nq.linear_noalloc_into(x, lay, y)
    assert e.value.status == nq.NQ_ERR_WORKSPACE
