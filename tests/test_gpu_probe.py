"""GPU: the read-rate probe reads every word of its buffer exactly once (the
XOR it returns equals the XOR of all words computed on the host), for one
batch, a single-launch size below the grid cap and a size that makes every
wave loop."""
import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("batches", [1, 3, 2238, 4096 + 77, 3 * 4096])
def test_read_probe_xor_of_all_words(batches):
    gen = torch.Generator().manual_seed(batches)
    host = torch.randint(-2**31, 2**31 - 1, (batches * 4096,), generator=gen, dtype=torch.int64).to(torch.int32)
    buf = host.to(G.DEV)
    sink = torch.zeros(1, dtype=torch.int32, device=G.DEV)
    wgs, thr = nq.read_probe(buf, sink)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(host.numpy().view(np.uint32))
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == int(want)
    assert thr == 256 and wgs == (min(batches, 4096) + 3) // 4
    # a second call XORs the same value again: back to zero
    nq.read_probe(buf, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0
