"""Seeded synthetic inputs for binary low-rank linear layers.

This module only draws random numbers and rounds them to storage dtypes.  It
holds none of the layer arithmetic, so that the fp64 oracle (``oracle/``) and
the HIP path (``binary_rank_gemv_packed_amd``) can both be fed from it without
sharing any computation.

Distributions (the pages give none; these are the plainest choice, as stated
in the workload descriptions of the Llama-shaped test layers):

* sign matrices ``U`` (m x r) and ``V`` (n x r): iid Bernoulli(1/2) over {-1, +1},
  stored as int8;
* scale vectors ``s1`` (m), ``g`` (r), ``s2`` (n): ``|N(0, 1)| + 0.1`` drawn in
  fp64, then rounded to the storage dtype (fp16 or fp32);
* activations ``x`` (B x n): ``N(0, 1)`` rounded to bf16 (or fp32).

Every tensor is drawn from its own stream,
``SeedSequence([20260206, cfg, block, layer, tensor_id])`` with PCG64, where
``tensor_id`` is 0 = U, 1 = V, 2 = s1, 3 = g, 4 = s2, 5 = x.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

ROOT_SEED = 20260206
TENSOR_IDS = {"U": 0, "V": 1, "s1": 2, "g": 3, "s2": 4, "x": 5}


def rng_for(cfg: int, block: int, layer: int, tensor: str) -> np.random.Generator:
    ss = np.random.SeedSequence([ROOT_SEED, cfg, block, layer, TENSOR_IDS[tensor]])
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); returns float32
    values that are exactly representable in bf16."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values already rounded to bf16."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def signs(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    return (rng.integers(0, 2, size=(rows, cols), dtype=np.int8) * 2 - 1).astype(np.int8)


def scales(rng: np.random.Generator, count: int, dtype) -> np.ndarray:
    v = np.abs(rng.standard_normal(count)) + 0.1
    return v.astype(dtype)


def activations(rng: np.random.Generator, rows: int, cols: int, dtype: str) -> np.ndarray:
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    if dtype == "bf16":
        return round_to_bf16(v)
    if dtype == "f32":
        return v
    raise ValueError(dtype)


@dataclass
class Layer:
    """One synthetic layer.  Scales are in their storage dtype (np.float16 or
    np.float32); ``x`` holds float32 values exactly representable in
    ``x_dtype``."""

    m: int
    n: int
    r: int
    U: np.ndarray
    V: np.ndarray
    s1: np.ndarray
    g: np.ndarray
    s2: np.ndarray
    x: np.ndarray
    x_dtype: str
    scale_dtype: str
    seed: tuple = field(default=())


def make_layer(m: int, n: int, r: int, B: int, *, cfg: int = 0, block: int = 0, layer: int = 0,
               scale_dtype: str = "f16", x_dtype: str = "bf16") -> Layer:
    sd = {"f16": np.float16, "f32": np.float32}[scale_dtype]
    U = signs(rng_for(cfg, block, layer, "U"), m, r)
    V = signs(rng_for(cfg, block, layer, "V"), n, r)
    s1 = scales(rng_for(cfg, block, layer, "s1"), m, sd)
    g = scales(rng_for(cfg, block, layer, "g"), r, sd)
    s2 = scales(rng_for(cfg, block, layer, "s2"), n, sd)
    x = activations(rng_for(cfg, block, layer, "x"), B, n, x_dtype)
    return Layer(m, n, r, U, V, s1, g, s2, x, x_dtype, scale_dtype, (ROOT_SEED, cfg, block, layer))


def make_integer_layer(m: int, n: int, r: int, B: int, *, seed: int = 0,
                       scale_dtype: str = "f32", x_dtype: str = "f32") -> Layer:
    """Layer whose every product and partial sum is an exact small dyadic
    rational: x in {-3..3}, s1, s2 in {1, 2}, g in {1, 1/2}."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, 99, seed])))
    sd = {"f16": np.float16, "f32": np.float32}[scale_dtype]
    U = signs(rng, m, r)
    V = signs(rng, n, r)
    s1 = rng.choice([1.0, 2.0], size=m).astype(sd)
    g = rng.choice([1.0, 0.5], size=r).astype(sd)
    s2 = rng.choice([1.0, 2.0], size=n).astype(sd)
    x = rng.integers(-3, 4, size=(B, n)).astype(np.float32)
    return Layer(m, n, r, U, V, s1, g, s2, x, x_dtype, scale_dtype, (ROOT_SEED, 99, seed))


# Llama-shaped layer shapes (out x in) and ranks at the bits/weight targets,
# from the rank rule applied with 16-bit scales.
LLAMA7B = {"q": (4096, 4096), "k": (4096, 4096), "v": (4096, 4096), "o": (4096, 4096),
           "gate": (11008, 4096), "up": (11008, 4096), "down": (4096, 11008)}
LLAMA70B = {"q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192), "o": (8192, 8192),
            "gate": (28672, 8192), "up": (28672, 8192), "down": (8192, 28672)}
LAYER_ORDER = ("q", "k", "v", "o", "gate", "up", "down")
