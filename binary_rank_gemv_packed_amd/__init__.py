"""Python binding of libnq: linear layers with a low-rank binary-factorised weight
W_hat = diag(s1) U diag(g) V^T diag(s2) on MI355X.

Argument marshalling only: every step of the forward runs in the HIP kernels of
libnq.so, reached through its C ABI (include/nq.h).  PyTorch provides device
memory and the current stream.  There is no CPU fallback: if the library is not
built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libnq.so")

NQ_OK, NQ_ERR_INVALID_ARG, NQ_ERR_NOT_PM1, NQ_ERR_WORKSPACE, NQ_ERR_UNSUPPORTED, NQ_ERR_HIP, NQ_ERR_INTERNAL = \
    0, -1, -2, -3, -4, -5, -6
NQ_F32, NQ_F16, NQ_BF16 = 0, 1, 2
NQ_GROUP_MAX = 4  # layers per group call (include/nq.h)
NQ_ENVELOPE_MAX = 4  # terms of a rank-l envelope (include/nq.h)
PATHS = {"auto": 0, "gemv": 1, "gemm": 2, "valu": 3, "decode": 4}

_DT = {torch.float32: NQ_F32, torch.float16: NQ_F16, torch.bfloat16: NQ_BF16}


class NQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libnq status {status}: {message}")
        self.status = status


class nq_layer(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("r", ctypes.c_int32),
                ("scale_dtype", ctypes.c_int32), ("blob", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libnq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing; build it with `python -m binary_rank_gemv_packed_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    c_int, c_size, vp = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    P = ctypes.POINTER(nq_layer)
    sigs = {
        "nq_abi_version": (c_int, []),
        "nq_layer_bytes": (c_size, [c_int, c_int, c_int, c_int]),
        "nq_pack_factors": (c_int, [P, vp, vp, vp, vp, vp, vp]),
        "nq_unpack_factors": (c_int, [P, vp, vp, vp]),
        "nq_transpose_layer": (c_int, [P, P, vp]),
        "nq_workspace_bytes": (c_size, [P, c_int]),
        "nq_workspace_bytes_path": (c_size, [P, c_int, c_int]),
        "nq_linear_fwd": (c_int, [P, vp, c_int, vp, c_int, c_int, vp, c_size, vp]),
        "nq_linear_fwd_path": (c_int, [P, vp, c_int, vp, c_int, c_int, vp, c_size, vp, c_int]),
        "nq_linear_fwd_profiled": (c_int, [P, vp, c_int, vp, c_int, c_int, vp, c_size, vp, c_int, vp, c_int,
                                           ctypes.POINTER(c_int), vp]),
        "nq_linear_fwd_noalloc": (c_int, [P, vp, c_int, vp, c_int, c_int, vp]),
        "nq_workspace_bytes_group": (c_size, [vp, c_int, c_int]),
        "nq_workspace_bytes_envelope": (c_size, [P, c_int, c_int]),
        "nq_linear_fwd_envelope": (c_int, [P, c_int, vp, vp, vp, c_int, vp, c_int, c_int, vp, c_size, vp]),
        "nq_linear_fwd_group": (c_int, [vp, c_int, vp, c_int, vp, c_int, c_int, vp, c_size, vp]),
        "nq_linear_fwd_group_profiled": (c_int, [vp, c_int, vp, c_int, vp, c_int, c_int, vp, c_size, vp, vp, c_int,
                                                 ctypes.POINTER(c_int), vp]),
        "nq_read_probe": (c_int, [vp, c_size, vp, vp, ctypes.POINTER(c_int)]),
        "nq_admm_workspace_bytes": (c_size, [c_int, c_int, c_int]),
        "nq_admm_factorize": (c_int, [vp, c_int, c_int, c_int, vp, vp, ctypes.c_float, c_int, c_int, vp, vp, vp, vp,
                                      vp, vp, vp, c_size, vp]),
        "nq_balance_scales": (c_int, [vp, vp, vp, c_int, c_int, c_int, vp]),
        "nq_bits_per_weight": (ctypes.c_double, [c_int, c_int, c_int, c_int]),
        "nq_rank_for_bits": (c_int, [c_int, c_int, ctypes.c_double, c_int]),
        "nq_status_string": (ctypes.c_char_p, [c_int]),
        "nq_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def _check(status: int) -> None:
    if status != NQ_OK:
        raise NQError(status, lib().nq_last_error().decode() or lib().nq_status_string(status).decode())


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class Layer:
    """A packed layer: the device blob plus its dimensions."""

    def __init__(self, m: int, n: int, r: int, scale_dtype: torch.dtype, blob: torch.Tensor):
        self.m, self.n, self.r = m, n, r
        self.scale_dtype = scale_dtype
        self.blob = blob
        self.c = nq_layer(m, n, r, _DT[scale_dtype], blob.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self.c)

    @property
    def device(self):
        return self.blob.device


def layer_bytes(m: int, n: int, r: int, scale_dtype: torch.dtype = torch.float16) -> int:
    return int(lib().nq_layer_bytes(m, n, r, _DT[scale_dtype]))


def empty_layer(m: int, n: int, r: int, scale_dtype: torch.dtype = torch.float16, device="cuda") -> Layer:
    nbytes = layer_bytes(m, n, r, scale_dtype)
    if nbytes == 0:
        raise NQError(NQ_ERR_INVALID_ARG, f"invalid layer dimensions m={m} n={n} r={r}")
    return Layer(m, n, r, scale_dtype, torch.empty(nbytes, dtype=torch.uint8, device=device))


def pack(U: torch.Tensor, V: torch.Tensor, s1: torch.Tensor, g: torch.Tensor, s2: torch.Tensor,
         stream=None) -> Layer:
    """Packs int8 sign matrices U (m x r), V (n x r) and scales (fp16 or fp32,
    all of one dtype) already on the GPU.  Blocks until validation is done."""
    m, r = U.shape
    n, r2 = V.shape
    if r2 != r or s1.shape != (m,) or g.shape != (r,) or s2.shape != (n,):
        raise NQError(NQ_ERR_INVALID_ARG, "shape mismatch between U, V and the scale vectors")
    if U.dtype != torch.int8 or V.dtype != torch.int8:
        raise NQError(NQ_ERR_INVALID_ARG, "U and V must be int8")
    if not (s1.dtype == g.dtype == s2.dtype) or s1.dtype not in (torch.float16, torch.float32):
        raise NQError(NQ_ERR_INVALID_ARG, "scales must share one dtype, fp16 or fp32")
    U, V, s1, g, s2 = (t.contiguous() for t in (U, V, s1, g, s2))
    layer = empty_layer(m, n, r, s1.dtype, U.device)
    _check(lib().nq_pack_factors(layer.ref, U.data_ptr(), V.data_ptr(), s1.data_ptr(), g.data_ptr(),
                                 s2.data_ptr(), _stream(stream)))
    return layer


def unpack(layer: Layer, stream=None):
    """Sign matrices (U, V) read back from the packed blob, as int8 +-1."""
    U = torch.empty((layer.m, layer.r), dtype=torch.int8, device=layer.device)
    V = torch.empty((layer.n, layer.r), dtype=torch.int8, device=layer.device)
    _check(lib().nq_unpack_factors(layer.ref, U.data_ptr(), V.data_ptr(), _stream(stream)))
    return U, V


def transpose(layer: Layer, stream=None) -> Layer:
    """The layer of W_hat^T (U and V, s1 and s2 swapped, factors bit-transposed
    on the GPU): linear(dy, transpose(layer)) = dy W_hat, the backward product."""
    out = empty_layer(layer.n, layer.m, layer.r, layer.scale_dtype, device=layer.device)
    _check(lib().nq_transpose_layer(layer.ref, out.ref, _stream(stream)))
    return out


def workspace_bytes(layer: Layer, B: int, path: str = "auto") -> int:
    return int(lib().nq_workspace_bytes_path(layer.ref, B, PATHS[path]))


def new_workspace(layer: Layer, B: int) -> torch.Tensor:
    return torch.empty(max(workspace_bytes(layer, B), 256), dtype=torch.uint8, device=layer.device)


def linear_into(x: torch.Tensor, layer: Layer, y: torch.Tensor, workspace: torch.Tensor, path: str = "auto",
                stream=None) -> torch.Tensor:
    """y[B, m] = x[B, n] W_hat^T into caller buffers; enqueues on the stream and
    returns without synchronising (safe to capture in a graph)."""
    B = x.shape[0] if x.dim() == 2 else 1
    if x.dtype not in (torch.bfloat16, torch.float32) or y.dtype not in (torch.bfloat16, torch.float32):
        raise NQError(NQ_ERR_INVALID_ARG, "x and y must be bf16 or fp32")
    if not (x.is_contiguous() and y.is_contiguous()):
        raise NQError(NQ_ERR_INVALID_ARG, "x and y must be contiguous")
    if x.numel() != B * layer.n or y.numel() != B * layer.m:
        raise NQError(NQ_ERR_INVALID_ARG, "x or y has the wrong number of elements")
    _check(lib().nq_linear_fwd_path(layer.ref, x.data_ptr(), _DT[x.dtype], y.data_ptr(), _DT[y.dtype], B,
                                    workspace.data_ptr(), workspace.numel(), _stream(stream), PATHS[path]))
    return y


def linear_into_profiled(x: torch.Tensor, layer: Layer, y: torch.Tensor, workspace: torch.Tensor, events,
                         path: str = "auto", stream=None):
    """linear_into that records the given HIP events (raw hipEvent_t handles, as
    ints) around each kernel launch.  Returns [(workgroups, threads per
    workgroup)] of the launches, in order."""
    B = x.shape[0] if x.dim() == 2 else 1
    arr = (ctypes.c_void_p * len(events))(*events)
    dims = (ctypes.c_int32 * (2 * len(events)))()
    nl = ctypes.c_int32(0)
    _check(lib().nq_linear_fwd_profiled(layer.ref, x.data_ptr(), _DT[x.dtype], y.data_ptr(), _DT[y.dtype], B,
                                        workspace.data_ptr(), workspace.numel(), _stream(stream), PATHS[path],
                                        ctypes.cast(arr, ctypes.c_void_p), len(events), ctypes.byref(nl),
                                        ctypes.cast(dims, ctypes.c_void_p)))
    k = min(nl.value, len(events) - 1)
    return [(dims[2 * i], dims[2 * i + 1]) for i in range(k)]


def _group_arrays(layers, ys=None):
    refs = (ctypes.POINTER(nq_layer) * len(layers))(*[ctypes.pointer(L.c) for L in layers])
    yp = None if ys is None else (ctypes.c_void_p * len(ys))(*[y.data_ptr() for y in ys])
    return refs, yp


def workspace_bytes_group(layers, B: int) -> int:
    refs, _ = _group_arrays(layers)
    return int(lib().nq_workspace_bytes_group(ctypes.cast(refs, ctypes.c_void_p), len(layers), B))


def _check_group(x, layers, ys):
    B = x.shape[0] if x.dim() == 2 else 1
    if len(ys) != len(layers):
        raise NQError(NQ_ERR_INVALID_ARG, "one output per layer")
    if x.dtype not in (torch.bfloat16, torch.float32) or any(y.dtype != ys[0].dtype for y in ys) or \
            ys[0].dtype not in (torch.bfloat16, torch.float32):
        raise NQError(NQ_ERR_INVALID_ARG, "x and the outputs must be bf16 or fp32 (one dtype for all outputs)")
    if not x.is_contiguous() or not all(y.is_contiguous() for y in ys):
        raise NQError(NQ_ERR_INVALID_ARG, "x and the outputs must be contiguous")
    if any(x.numel() != B * L.n for L in layers) or any(y.numel() != B * L.m for y, L in zip(ys, layers)):
        raise NQError(NQ_ERR_INVALID_ARG, "x or an output has the wrong number of elements")
    return B


def linear_group_into(x: torch.Tensor, layers, ys, workspace: torch.Tensor, stream=None):
    """ys[l] = x W_hat_l^T for layers sharing x (q/k/v, gate/up): two launches
    in all for B <= 4 (stage 1 over every layer's V^T, block-diagonal stage 2)."""
    B = _check_group(x, layers, ys)
    refs, yp = _group_arrays(layers, ys)
    _check(lib().nq_linear_fwd_group(ctypes.cast(refs, ctypes.c_void_p), len(layers), x.data_ptr(), _DT[x.dtype],
                                     ctypes.cast(yp, ctypes.c_void_p), _DT[ys[0].dtype], B, workspace.data_ptr(),
                                     workspace.numel(), _stream(stream)))
    return ys


def linear_group(x: torch.Tensor, layers, out_dtype: torch.dtype | None = None, stream=None):
    xx = x if x.dim() == 2 else x.view(1, -1)
    ys = [torch.empty((xx.shape[0], L.m), dtype=out_dtype or x.dtype, device=x.device) for L in layers]
    ws = torch.empty(max(workspace_bytes_group(layers, xx.shape[0]), 256), dtype=torch.uint8, device=x.device)
    linear_group_into(xx, layers, ys, ws, stream)
    return ys if x.dim() == 2 else [y.view(-1) for y in ys]


def linear_group_into_profiled(x: torch.Tensor, layers, ys, workspace: torch.Tensor, events, stream=None):
    """linear_group_into that records HIP events around each launch; returns
    [(workgroups, threads per workgroup)] of the launches."""
    B = _check_group(x, layers, ys)
    refs, yp = _group_arrays(layers, ys)
    arr = (ctypes.c_void_p * len(events))(*events)
    dims = (ctypes.c_int32 * (2 * len(events)))()
    nl = ctypes.c_int32(0)
    _check(lib().nq_linear_fwd_group_profiled(ctypes.cast(refs, ctypes.c_void_p), len(layers), x.data_ptr(),
                                              _DT[x.dtype], ctypes.cast(yp, ctypes.c_void_p), _DT[ys[0].dtype], B,
                                              workspace.data_ptr(), workspace.numel(), _stream(stream),
                                              ctypes.cast(arr, ctypes.c_void_p), len(events), ctypes.byref(nl),
                                              ctypes.cast(dims, ctypes.c_void_p)))
    k = min(nl.value, len(events) - 1)
    return [(dims[2 * i], dims[2 * i + 1]) for i in range(k)]


def linear_envelope(x: torch.Tensor, layer: Layer, s1_env: torch.Tensor, s2_env: torch.Tensor,
                    out_dtype: torch.dtype | None = None, stream=None) -> torch.Tensor:
    """y = x W_hat^T with W_hat = sum_t diag(s1_env[t]) U diag(g) V^T diag(s2_env[t])
    (rank-l envelope; U, V, g from the layer): B x terms <= 4."""
    xx = x if x.dim() == 2 else x.view(1, -1)
    B, env = xx.shape[0], s1_env.shape[0]
    if s1_env.shape != (env, layer.m) or s2_env.shape != (env, layer.n) or \
            s1_env.dtype != layer.scale_dtype or s2_env.dtype != layer.scale_dtype:
        raise NQError(NQ_ERR_INVALID_ARG, "envelope scales must be (terms, m) and (terms, n) in the layer's dtype")
    if not (xx.is_contiguous() and s1_env.is_contiguous() and s2_env.is_contiguous()):
        raise NQError(NQ_ERR_INVALID_ARG, "x and the envelope scales must be contiguous")
    y = torch.empty((B, layer.m), dtype=out_dtype or x.dtype, device=x.device)
    ws = torch.empty(max(int(lib().nq_workspace_bytes_envelope(layer.ref, env, B)), 256), dtype=torch.uint8,
                     device=x.device)
    _check(lib().nq_linear_fwd_envelope(layer.ref, env, s1_env.data_ptr(), s2_env.data_ptr(), xx.data_ptr(),
                                        _DT[xx.dtype], y.data_ptr(), _DT[y.dtype], B, ws.data_ptr(), ws.numel(),
                                        _stream(stream)))
    return y if x.dim() == 2 else y.view(-1)


def linear_noalloc_into(x: torch.Tensor, layer: Layer, y: torch.Tensor, stream=None) -> torch.Tensor:
    """linear_into without a workspace: the library's static device scratch is
    used (see nq_linear_fwd_noalloc; calls overlapping on one GPU race)."""
    B = x.shape[0] if x.dim() == 2 else 1
    if x.dtype not in (torch.bfloat16, torch.float32) or y.dtype not in (torch.bfloat16, torch.float32):
        raise NQError(NQ_ERR_INVALID_ARG, "x and y must be bf16 or fp32")
    if not (x.is_contiguous() and y.is_contiguous()):
        raise NQError(NQ_ERR_INVALID_ARG, "x and y must be contiguous")
    if x.numel() != B * layer.n or y.numel() != B * layer.m:
        raise NQError(NQ_ERR_INVALID_ARG, "x or y has the wrong number of elements")
    _check(lib().nq_linear_fwd_noalloc(layer.ref, x.data_ptr(), _DT[x.dtype], y.data_ptr(), _DT[y.dtype], B,
                                       _stream(stream)))
    return y


def linear(x: torch.Tensor, layer: Layer, out_dtype: torch.dtype | None = None, path: str = "auto",
           workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """y = x W_hat^T for x of shape (B, n) or (n,); y has x's dtype unless given."""
    squeeze = x.dim() == 1
    x2 = x.reshape(1, -1) if squeeze else x
    x2 = x2.contiguous()
    B = x2.shape[0]
    y = torch.empty((B, layer.m), dtype=out_dtype or x.dtype, device=x.device)
    if workspace is None:
        workspace = new_workspace(layer, B)
    linear_into(x2, layer, y, workspace, path, stream)
    return y[0] if squeeze else y


def read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> tuple[int, int]:
    """Reads buf once (a measurement aid; see nq_read_probe) and XORs its
    32-bit words into sink[0] (int32, on buf's device).  Returns the launch's
    (workgroups, threads per workgroup)."""
    if not buf.is_contiguous() or sink.dtype != torch.int32 or sink.numel() < 1:
        raise NQError(NQ_ERR_INVALID_ARG, "buf must be contiguous and sink an int32 tensor")
    grid = (ctypes.c_int32 * 2)()
    _check(lib().nq_read_probe(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(), _stream(stream),
                               grid))
    return int(grid[0]), int(grid[1])


def admm_factorize(W: torch.Tensor, A0: torch.Tensor, B0: torch.Tensor, rho: float, iters: int,
                   power_iters: int, with_err: bool = True, stream=None):
    """Initialiser of the binary factors of a dense fp32 weight W (m x n) from
    latent factors A0 (m x r), B0 (n x r), all on the GPU (nq_admm_factorize).
    Returns (U int8 m x r, V int8 n x r, s1, g, s2 fp32, err fp32 [iters + 1]
    or None)."""
    m, n = W.shape
    r = A0.shape[1]
    if A0.shape != (m, r) or B0.shape != (n, r):
        raise NQError(NQ_ERR_INVALID_ARG, f"A0 {tuple(A0.shape)} / B0 {tuple(B0.shape)} do not match W {m}x{n}, r={r}")
    for t in (W, A0, B0):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise NQError(NQ_ERR_INVALID_ARG, "W, A0 and B0 must be contiguous fp32 GPU tensors")
    dev = W.device
    need = int(lib().nq_admm_workspace_bytes(m, n, r))
    if need == 0:
        raise NQError(NQ_ERR_INVALID_ARG, f"invalid dimensions m={m} n={n} r={r}")
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    U = torch.empty(m, r, dtype=torch.int8, device=dev)
    V = torch.empty(n, r, dtype=torch.int8, device=dev)
    s1 = torch.empty(m, dtype=torch.float32, device=dev)
    g = torch.empty(r, dtype=torch.float32, device=dev)
    s2 = torch.empty(n, dtype=torch.float32, device=dev)
    err = torch.empty(iters + 1, dtype=torch.float32, device=dev) if with_err else None
    _check(lib().nq_admm_factorize(W.data_ptr(), m, n, r, A0.data_ptr(), B0.data_ptr(), float(rho), iters,
                                   power_iters, U.data_ptr(), V.data_ptr(), s1.data_ptr(), g.data_ptr(),
                                   s2.data_ptr(), err.data_ptr() if err is not None else None, ws.data_ptr(),
                                   ws.numel(), _stream(stream)))
    return U, V, s1, g, s2, err


def balance_scales(s1: torch.Tensor, g: torch.Tensor, s2: torch.Tensor, stream=None) -> None:
    """Power-of-two magnitude balancing of fp32 GPU scale vectors, in place
    (nq_balance_scales)."""
    for t in (s1, g, s2):
        if t.dtype != torch.float32 or not t.is_contiguous() or not t.is_cuda:
            raise NQError(NQ_ERR_INVALID_ARG, "s1, g and s2 must be contiguous fp32 GPU tensors")
    _check(lib().nq_balance_scales(s1.data_ptr(), g.data_ptr(), s2.data_ptr(), s1.numel(), s2.numel(), g.numel(),
                                   _stream(stream)))


def bits_per_weight(m: int, n: int, r: int, scale_bits: int = 16) -> float:
    return float(lib().nq_bits_per_weight(m, n, r, scale_bits))


def rank_for_bits(m: int, n: int, bpw: float, scale_bits: int = 16) -> int:
    return int(lib().nq_rank_for_bits(m, n, bpw, scale_bits))


def abi_version() -> int:
    return int(lib().nq_abi_version())
