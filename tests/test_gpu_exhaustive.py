"""Every sign pattern of tiny layers through the C ABI (pack + forward), with
small-integer activations and dyadic scales, so that the GPU result must equal
the fp64 oracle exactly.  Checks every bit position of the packed layout, the
bit-to-sign convention (bit 1 = +1) and both sign-matrix products at once."""
import itertools

import numpy as np
import pytest
import torch

import binary_rank_gemv_packed_amd as nq
from oracle import nq_oracle as O
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

SHAPES = [(1, 1, 1), (2, 2, 1), (2, 3, 1), (3, 3, 2), (2, 2, 3)]


def _patterns(m, n, r):
    nb = r * (m + n)
    for code in range(2 ** nb):
        bits = np.array([(code >> i) & 1 for i in range(nb)], np.int8) * 2 - 1
        yield bits[: m * r].reshape(m, r), bits[m * r:].reshape(n, r)


@pytest.mark.parametrize("m,n,r", SHAPES)
@pytest.mark.parametrize("path", ["decode", "gemv"])
def test_every_sign_pattern_exact(m, n, r, path):
    rng = np.random.default_rng(100 + 10 * m + n + r)
    B = 2
    x = rng.integers(-3, 4, size=(B, n)).astype(np.float32)
    x[0, 0] = 1.0  # at least one non-zero activation
    s1 = rng.choice([1.0, 2.0, 0.5], m).astype(np.float32)
    g = rng.choice([1.0, 2.0, 0.5], r).astype(np.float32)
    s2 = rng.choice([1.0, 2.0, 0.5], n).astype(np.float32)
    xt = torch.from_numpy(x).to(G.DEV)
    t1, tg, t2 = (torch.from_numpy(a).to(G.DEV) for a in (s1, g, s2))
    pats = list(_patterns(m, n, r))
    Uall = torch.from_numpy(np.stack([p[0] for p in pats])).to(G.DEV)
    Vall = torch.from_numpy(np.stack([p[1] for p in pats])).to(G.DEV)
    ys = []
    ws = None
    for i in range(len(pats)):
        layer = nq.pack(Uall[i], Vall[i], t1, tg, t2)
        if ws is None:
            ws = nq.new_workspace(layer, B)
        ys.append(nq.linear(xt, layer, out_dtype=torch.float32, path=path, workspace=ws))
    y = torch.stack(ys).cpu().numpy().astype(np.float64)
    bad = 0
    for i, (U, V) in enumerate(pats):
        ref = O.linear_dense(x.astype(np.float64), U, V, s1, g, s2)
        if not np.array_equal(y[i], ref):
            bad += 1
    assert bad == 0, f"{bad} of {len(pats)} sign patterns differ from the oracle"
