"""C ABI checks that need no GPU: exports, sizes, accounting, and every
argument-validation error path (validation happens before any HIP call)."""
import ctypes
import os
import re

import pytest

import binary_rank_gemv_packed_amd as nq
from oracle import nq_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x7F0000000000  # 256-aligned pointer value that is never dereferenced


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(nq.LIB_PATH):
        from binary_rank_gemv_packed_amd import build
        build.build()
    return nq.lib()


def header_functions():
    text = open(os.path.join(ROOT, "include", "nq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nq_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert len(names) >= 11
    for name in names:
        assert hasattr(L, name), name


def test_version(L):
    assert nq.abi_version() == 1


def _layout_bytes(m, n, r, sb):
    """The blob layout as documented in include/nq.h and csrc/nq_common.h."""
    up = lambda v: (v + 255) // 256 * 256
    tiles = lambda R, C: ((R + 15) // 16) * ((C + 127) // 128) * 256
    o = 256
    o = up(o + tiles(m, r))
    o = up(o + tiles(r, n))
    o = up(o + m * sb)
    o = up(o + r * sb)
    return up(o + n * sb)


@pytest.mark.parametrize("m,n,r,dt,sb", [(256, 256, 64, nq.NQ_F32, 4), (63, 17, 5, nq.NQ_F16, 2),
                                         (28672, 8192, 5079, nq.NQ_F16, 2), (1, 1, 1, nq.NQ_F16, 2)])
def test_layer_bytes(L, m, n, r, dt, sb):
    assert L.nq_layer_bytes(m, n, r, dt) == _layout_bytes(m, n, r, sb)


def test_layer_bytes_invalid(L):
    assert L.nq_layer_bytes(0, 5, 5, nq.NQ_F16) == 0
    assert L.nq_layer_bytes(5, 5, 0, nq.NQ_F16) == 0
    assert L.nq_layer_bytes(5, 5, 5, nq.NQ_BF16) == 0
    assert L.nq_layer_bytes(5, (1 << 20) + 1, 5, nq.NQ_F16) == 0


@pytest.mark.parametrize("m,n,r", [(256, 256, 64), (4096, 11008, 2369), (7, 3, 100), (1, 1, 0)])
@pytest.mark.parametrize("bits", [0, 16, 32])
def test_bits_per_weight_agrees_with_oracle(L, m, n, r, bits):
    assert nq.bits_per_weight(m, n, r, bits) == O.bits_per_weight(m, n, r, bits)


@pytest.mark.parametrize("m,n", [(4096, 4096), (11008, 4096), (1024, 8192), (28672, 8192), (63, 17), (1, 1)])
@pytest.mark.parametrize("bpw", [0.3, 0.55, 0.8, 1.0, 4.0])
def test_rank_for_bits_agrees_with_oracle(L, m, n, bpw):
    assert nq.rank_for_bits(m, n, bpw, 16) == O.rank_for_bits(m, n, bpw, 16)


def test_rank_for_bits_invalid(L):
    assert nq.rank_for_bits(0, 4, 1.0) == -1
    assert nq.rank_for_bits(4, 4, -1.0) == -1
    assert nq.bits_per_weight(0, 4, 1) == -1.0


def _layer(m=64, n=96, r=40, dt=nq.NQ_F16, blob=FAKE):
    return nq.nq_layer(m, n, r, dt, blob)


def fwd(L, layer, x=FAKE, xdt=nq.NQ_BF16, y=FAKE + (1 << 30), ydt=nq.NQ_BF16, B=1, ws=FAKE + (2 << 30),
        wsb=1 << 30, path=0):
    ref = ctypes.byref(layer) if layer is not None else None
    return L.nq_linear_fwd_path(ref, x, xdt, y, ydt, B, ws, wsb, None, path)


def test_fwd_validation_errors(L):
    E = nq
    assert fwd(L, None) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(m=0)) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(r=70000)) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(dt=nq.NQ_BF16)) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(blob=0)) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(blob=FAKE + 16)) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), B=-1) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), xdt=nq.NQ_F16) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), ydt=7) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), x=0) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), y=0) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), x=FAKE + 1) == E.NQ_ERR_INVALID_ARG           # misaligned bf16
    assert fwd(L, _layer(), y=FAKE + 2, ydt=nq.NQ_F32) == E.NQ_ERR_INVALID_ARG  # misaligned f32
    assert fwd(L, _layer(), y=FAKE + 64) == E.NQ_ERR_INVALID_ARG          # overlaps x
    assert fwd(L, _layer(), path=9) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), wsb=16) == E.NQ_ERR_WORKSPACE
    assert fwd(L, _layer(), ws=0) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), ws=FAKE + (2 << 30) + 128) == E.NQ_ERR_INVALID_ARG
    assert fwd(L, _layer(), B=17, path=nq.PATHS["gemv"]) == E.NQ_ERR_UNSUPPORTED
    assert fwd(L, _layer(), B=2, path=nq.PATHS["valu"]) == E.NQ_ERR_UNSUPPORTED
    assert b"overlap" not in L.nq_last_error()
    fwd(L, _layer(), y=FAKE + 64)
    assert b"overlap" in L.nq_last_error()


def test_fwd_batch_zero_is_a_no_op(L):
    # valid arguments, nothing to do: returns before any HIP call
    assert fwd(L, _layer(), B=0, x=0, y=0) == nq.NQ_OK


def test_workspace_bytes(L):
    lay = _layer(m=28672, n=8192, r=5079)
    ref = ctypes.byref(lay)
    assert L.nq_workspace_bytes(ref, 0) == 0
    assert L.nq_workspace_bytes(None, 1) == 0
    w1 = L.nq_workspace_bytes(ref, 1)
    assert 0 < w1 < 64 << 20
    assert fwd(L, lay, wsb=w1 - 1) == nq.NQ_ERR_WORKSPACE


def test_pack_validation_errors(L):
    lay = _layer()
    ref = ctypes.byref(lay)
    assert L.nq_pack_factors(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == nq.NQ_ERR_INVALID_ARG
    assert L.nq_pack_factors(ref, 0, FAKE, FAKE, FAKE, FAKE, None) == nq.NQ_ERR_INVALID_ARG
    assert L.nq_pack_factors(ref, FAKE, FAKE, FAKE, 0, FAKE, None) == nq.NQ_ERR_INVALID_ARG
    bad = _layer(blob=FAKE + 8)
    assert L.nq_pack_factors(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, FAKE, None) == nq.NQ_ERR_INVALID_ARG
    assert L.nq_unpack_factors(ref, 0, FAKE, None) == nq.NQ_ERR_INVALID_ARG


def test_status_strings(L):
    for s in (0, -1, -2, -3, -4, -5, -6):
        assert L.nq_status_string(s)
    assert L.nq_status_string(42) == b"unknown status"
