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
PATHS = {"auto": 0, "gemv": 1, "gemm": 2, "valu": 3}

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
        "nq_workspace_bytes": (c_size, [P, c_int]),
        "nq_linear_fwd": (c_int, [P, vp, c_int, vp, c_int, c_int, vp, c_size, vp]),
        "nq_linear_fwd_path": (c_int, [P, vp, c_int, vp, c_int, c_int, vp, c_size, vp, c_int]),
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


def workspace_bytes(layer: Layer, B: int) -> int:
    return int(lib().nq_workspace_bytes(layer.ref, B))


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


def bits_per_weight(m: int, n: int, r: int, scale_bits: int = 16) -> float:
    return float(lib().nq_bits_per_weight(m, n, r, scale_bits))


def rank_for_bits(m: int, n: int, bpw: float, scale_bits: int = 16) -> int:
    return int(lib().nq_rank_for_bits(m, n, bpw, scale_bits))


def abi_version() -> int:
    return int(lib().nq_abi_version())
