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
    assert fwd(L, _layer(), B=17, path=nq.PATHS["decode"]) == E.NQ_ERR_UNSUPPORTED
    assert fwd(L, _layer(), B=17, wsb=16) == E.NQ_ERR_WORKSPACE   # B > 16: the prefill path's workspace
    assert b"overlap" not in L.nq_last_error()
    fwd(L, _layer(), y=FAKE + 64)
    assert b"overlap" in L.nq_last_error()


def test_noalloc_validation_before_any_hip_call(L):
    big = _layer(m=8192, n=28672, r=5079)
    # 2048 tokens need far more than the 16 MiB static scratch: refused on the host
    assert L.nq_linear_fwd_noalloc(ctypes.byref(big), FAKE, nq.NQ_BF16, FAKE + (1 << 30), nq.NQ_BF16, 2048,
                                   None) == nq.NQ_ERR_WORKSPACE
    assert b"16777216" in L.nq_last_error()
    assert L.nq_linear_fwd_noalloc(None, FAKE, nq.NQ_BF16, FAKE, nq.NQ_BF16, 1, None) == nq.NQ_ERR_INVALID_ARG
    assert L.nq_linear_fwd_noalloc(ctypes.byref(big), FAKE, nq.NQ_BF16, FAKE, nq.NQ_BF16, -1, None) == \
        nq.NQ_ERR_INVALID_ARG


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
    for name in ("decode", "gemv", "valu"):
        need = L.nq_workspace_bytes_path(ref, 1, nq.PATHS[name])
        assert 0 < need <= w1
        assert fwd(L, lay, wsb=need - 1, path=nq.PATHS[name]) == nq.NQ_ERR_WORKSPACE
    assert L.nq_workspace_bytes_path(ref, 17, nq.PATHS["decode"]) == 0
    # B = 5..16 runs as chunks of 4 rows: the workspace of one chunk
    assert L.nq_workspace_bytes_path(ref, 16, nq.PATHS["decode"]) == L.nq_workspace_bytes_path(ref, 4, nq.PATHS["decode"])
    assert L.nq_workspace_bytes_path(ref, 17, nq.PATHS["gemv"]) == 0
    assert L.nq_workspace_bytes_path(ref, 2, nq.PATHS["valu"]) == 0
    assert L.nq_workspace_bytes_path(ref, 1, 99) == 0
    # prefill: X' fp16 + T fp32 + T' fp16 for 2048 tokens
    big = L.nq_workspace_bytes_path(ref, 2048, nq.PATHS["gemm"])
    assert big >= 2048 * (64 * 128 * 2 + 5079 * 4 + 40 * 128 * 2)
    assert L.nq_workspace_bytes(ref, 2048) == big


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


# ------------------------------------------------------------------ layer groups
def _group(layers):
    return ctypes.cast((ctypes.POINTER(nq.nq_layer) * len(layers))(*[ctypes.pointer(l) for l in layers]),
                       ctypes.c_void_p)


def _ptrs(vals):
    return ctypes.cast((ctypes.c_void_p * len(vals))(*vals), ctypes.c_void_p)


def test_group_validation(L):
    q, k = _layer(m=8192, n=8192, r=3257), _layer(m=1024, n=8192, r=710)
    other_n = _layer(m=1024, n=4096, r=710)
    ys = _ptrs([FAKE + (1 << 30), FAKE + (2 << 30)])
    ws = L.nq_workspace_bytes_group(_group([q, k]), 2, 1)
    assert ws > 0
    run = lambda grp, n, yp, B=1, wsb=ws: L.nq_linear_fwd_group(grp, n, FAKE, nq.NQ_BF16, yp, nq.NQ_BF16, B, FAKE,
                                                                wsb, None)
    assert run(_group([q, k]), 0, ys) == nq.NQ_ERR_INVALID_ARG
    assert run(_group([q, k]), nq.NQ_GROUP_MAX + 1, ys) == nq.NQ_ERR_INVALID_ARG
    assert run(_group([q, other_n]), 2, ys) == nq.NQ_ERR_INVALID_ARG
    assert b"shares x" in L.nq_last_error()
    assert run(_group([q, k]), 2, _ptrs([FAKE + (1 << 30), FAKE + (1 << 30) + 64])) == nq.NQ_ERR_INVALID_ARG
    assert b"overlap" in L.nq_last_error()
    assert run(_group([q, k]), 2, _ptrs([FAKE, FAKE + (2 << 30)])) == nq.NQ_ERR_INVALID_ARG  # ys[0] on x
    assert run(_group([q, k]), 2, ys, wsb=ws - 1) == nq.NQ_ERR_WORKSPACE
    assert run(_group([q, k]), 2, ys, B=0) == nq.NQ_OK
    assert L.nq_workspace_bytes_group(_group([q, other_n]), 2, 1) == 0


def test_group_workspace_covers_the_fallback(L):
    q, k = _layer(m=8192, n=8192, r=3257), _layer(m=1024, n=8192, r=710)
    for B in (5, 16, 17, 2048):  # beyond the fused path: the layers run one after another
        need = max(L.nq_workspace_bytes_path(ctypes.byref(l), B, 0) for l in (q, k))
        assert L.nq_workspace_bytes_group(_group([q, k]), 2, B) <= need
        assert L.nq_workspace_bytes_group(_group([q, k]), 2, B) > 0


def test_transpose_validation(L):
    src = _layer(m=64, n=96, r=40)
    good = _layer(m=96, n=64, r=40, blob=FAKE + (1 << 30))
    t = lambda s, d: L.nq_transpose_layer(ctypes.byref(s) if s is not None else None,
                                          ctypes.byref(d) if d is not None else None, None)
    assert t(None, good) == nq.NQ_ERR_INVALID_ARG
    assert t(src, None) == nq.NQ_ERR_INVALID_ARG
    assert t(src, _layer(m=64, n=96, r=40, blob=FAKE + (1 << 30))) == nq.NQ_ERR_INVALID_ARG  # not the transpose
    assert t(src, _layer(m=96, n=64, r=41, blob=FAKE + (1 << 30))) == nq.NQ_ERR_INVALID_ARG
    assert t(src, _layer(m=96, n=64, r=40, dt=nq.NQ_F32, blob=FAKE + (1 << 30))) == nq.NQ_ERR_INVALID_ARG
    assert t(src, _layer(m=96, n=64, r=40, blob=FAKE + 256)) == nq.NQ_ERR_INVALID_ARG  # blobs overlap
    assert b"overlap" in L.nq_last_error()


def test_envelope_validation(L):
    lay = _layer(m=64, n=96, r=40)
    ws = L.nq_workspace_bytes_envelope(ctypes.byref(lay), 2, 1)
    assert ws > 0
    assert L.nq_workspace_bytes_envelope(ctypes.byref(lay), 2, 3) == 0  # 6 batch rows: not this path
    assert L.nq_workspace_bytes_envelope(ctypes.byref(lay), 0, 1) == 0
    S1, S2, X, Y, W = FAKE + (3 << 30), FAKE + (4 << 30), FAKE, FAKE + (1 << 30), FAKE + (2 << 30)
    run = lambda env=2, B=1, s1=S1, s2=S2, wsb=ws: L.nq_linear_fwd_envelope(
        ctypes.byref(lay), env, s1, s2, X, nq.NQ_BF16, Y, nq.NQ_BF16, B, W, wsb, None)
    assert run(env=0) == nq.NQ_ERR_INVALID_ARG
    assert run(env=nq.NQ_ENVELOPE_MAX + 1) == nq.NQ_ERR_INVALID_ARG
    assert run(s1=0) == nq.NQ_ERR_INVALID_ARG
    assert run(s2=S2 + 1) == nq.NQ_ERR_INVALID_ARG  # misaligned fp16 array
    assert run(B=3) == nq.NQ_ERR_UNSUPPORTED
    assert run(wsb=ws - 1) == nq.NQ_ERR_WORKSPACE
    assert run(B=0) == nq.NQ_OK


def test_read_probe_validation(L):
    sink = FAKE + (1 << 30)
    probe = lambda buf=FAKE, nbytes=16384, s=sink: L.nq_read_probe(buf, nbytes, s, None, None)
    assert probe(buf=0) == nq.NQ_ERR_INVALID_ARG
    assert probe(s=0) == nq.NQ_ERR_INVALID_ARG
    assert probe(nbytes=0) == nq.NQ_ERR_INVALID_ARG
    assert probe(nbytes=16384 + 16) == nq.NQ_ERR_INVALID_ARG  # not a whole number of 16 KiB batches
    assert probe(buf=FAKE + 8) == nq.NQ_ERR_INVALID_ARG
    assert probe(s=sink + 2) == nq.NQ_ERR_INVALID_ARG
    assert probe(s=FAKE + 4096) == nq.NQ_ERR_INVALID_ARG  # sink inside buf
    assert b"inside" in L.nq_last_error()


def test_admm_validation(L):
    ws_need = L.nq_admm_workspace_bytes(64, 48, 8)
    assert ws_need > 0
    assert L.nq_admm_workspace_bytes(64, 48, 49) == 0  # r > min(m, n)
    assert L.nq_admm_workspace_bytes(0, 48, 8) == 0
    assert L.nq_admm_workspace_bytes(1 << 20, 1 << 20, 4096) == 0  # max(m, n) x r >= 2^31
    P = FAKE
    args = dict(W=P, m=64, n=48, r=8, A0=P, B0=P, rho=1.0, iters=2, K=3, U=P, V=P, s1=P, g=P, s2=P, err=None,
                ws=P, wsb=ws_need)

    def call(**kw):
        a = dict(args, **kw)
        return L.nq_admm_factorize(a["W"], a["m"], a["n"], a["r"], a["A0"], a["B0"], a["rho"], a["iters"], a["K"],
                                   a["U"], a["V"], a["s1"], a["g"], a["s2"], a["err"], a["ws"], a["wsb"], None)
    assert call(W=None) == nq.NQ_ERR_INVALID_ARG
    assert call(s2=None) == nq.NQ_ERR_INVALID_ARG
    assert call(r=49) == nq.NQ_ERR_INVALID_ARG
    assert call(m=1 << 20, n=1 << 19, r=4096) == nq.NQ_ERR_INVALID_ARG
    assert call(rho=0.0) == nq.NQ_ERR_INVALID_ARG
    assert call(rho=float("nan")) == nq.NQ_ERR_INVALID_ARG
    assert call(iters=-1) == nq.NQ_ERR_INVALID_ARG
    assert call(K=1001) == nq.NQ_ERR_INVALID_ARG
    assert call(W=P + 2) == nq.NQ_ERR_INVALID_ARG
    assert call(ws=P + 16) == nq.NQ_ERR_INVALID_ARG
    assert call(wsb=ws_need - 1) == nq.NQ_ERR_WORKSPACE
    assert b"workspace" in L.nq_last_error()
    assert L.nq_balance_scales(None, P, P, 4, 4, 2, None) == nq.NQ_ERR_INVALID_ARG
    assert L.nq_balance_scales(P, P, P, 0, 4, 2, None) == nq.NQ_ERR_INVALID_ARG
