"""Helpers for GPU tests: moving synthetic layers to the device and comparing
against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import binary_rank_gemv_packed_amd as nq
from oracle import nq_oracle as O

DEV = "cuda:0"
TOL = 2e-3  # relative L2 bar for bf16 activations with fp32 accumulation


def to_torch_scale(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def x_tensor(x: np.ndarray, x_dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)
    return t.to(torch.bfloat16) if x_dtype == "bf16" else t


def pack_layer(L) -> nq.Layer:
    return nq.pack(torch.from_numpy(L.U).to(DEV), torch.from_numpy(L.V).to(DEV), to_torch_scale(L.s1),
                   to_torch_scale(L.g), to_torch_scale(L.s2))


def rel_l2(y, ref) -> float:
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))


def run(L, layer=None, B=None, y_dtype=torch.bfloat16, path="auto", x_override=None):
    layer = layer or pack_layer(L)
    x = L.x if x_override is None else x_override
    xt = x_tensor(x, L.x_dtype)
    y = nq.linear(xt, layer, out_dtype=y_dtype, path=path)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def oracle(L, mode="dense", x=None):
    x = L.x if x is None else x
    f = O.linear_dense if mode == "dense" else O.linear_factored
    return f(x.astype(np.float64), L.U, L.V, L.s1.astype(np.float64), L.g.astype(np.float64),
             L.s2.astype(np.float64))


def bf16_round(a: np.ndarray) -> np.ndarray:
    """Round fp64 values to bf16 (nearest, ties to even) via fp32."""
    import synth
    return synth.round_to_bf16(np.asarray(a, np.float32).astype(np.float32)).astype(np.float64)


def bf16_ulp(a: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at the magnitude of each value (8 significand bits)."""
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def check_bf16_output(ybf, ref, y32=None, tol=TOL):
    """bf16 output against the fp64 oracle.

    * With the same call's fp32 output y32 (the kernels round their fp32 result
      once, to nearest even): ybf must be exactly bf16(y32), bit for bit.
    * Per element: |ybf - bf16(ref)| <= 1 bf16 ulp + 2 |y32 - ref|.  A plain
      one-ulp bar is wrong for outputs near zero, where the fp32 sum's absolute
      error (bounded in relative L2 by the fp32 check) exceeds that element's
      bf16 ulp; the fp32 error term covers exactly that.
    * Whole output: relative L2 within the tolerance plus the error that
      rounding the exact result to bf16 costs by itself."""
    ybf = np.asarray(ybf, np.float64)
    rref = bf16_round(ref)
    if y32 is not None:
        y32 = np.asarray(y32, np.float64)
        assert np.array_equal(ybf, bf16_round(y32))
        slack = bf16_ulp(rref) * (1 + 1e-9) + 2.0 * np.abs(y32 - ref)
        diff = np.abs(ybf - rref)
        assert np.all(diff <= slack), float(np.max(diff / slack))
    assert rel_l2(ybf, ref) <= tol + rel_l2(rref, ref)
