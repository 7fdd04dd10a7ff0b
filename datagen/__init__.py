"""Seeded synthetic inputs shaped like the pages' layers.

This module holds no quantization arithmetic: it only draws random tensors
(numpy PCG64 streams), shapes them and casts fp32 to bf16 bit patterns with
round-to-nearest-even.  Both the HIP path's tests/benchmark and the CPU oracle
take their inputs from here, and from nowhere else.

Recipes (seed per tensor):
  tiny     W 256x256 N(0,1) (seed 0), A 64x256 N(0,1) (seed 1), fp32
  sweep    4096x4096 fp32, N(0,1) (seed 2) and Student-t nu=3 (seed 3)
  mxfp4    X 4096x4096 N(0,1) (seed 4) with 8 channels x50 (chosen by seed 5),
           bf16; W 14336x4096 N(0, 0.02) (seed 6) fp32
  razer    W 17408x5120 N(0, 0.02) (seed 7) fp32; A M x 5120 Student-t nu=4,
           M in {1, 16, 128} (seeds 8, 9, 10), bf16
  prefill  A 32768x5120 Student-t nu=4 (seed 11) bf16; W N x 5120 N(0, 0.02)
           for N = 10240, 17408, 5120 (seeds 12, 13, 14) fp32
"""
from __future__ import annotations

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal(shape, seed: int, std: float = 1.0) -> np.ndarray:
    return (rng(seed).standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def student_t(shape, seed: int, nu: float) -> np.ndarray:
    return rng(seed).standard_t(nu, size=shape).astype(np.float32)


def with_outlier_channels(x: np.ndarray, seed: int, count: int = 8, factor: float = 50.0):
    """Scale `count` distinct random columns by `factor`; returns (x', columns)."""
    cols = np.sort(rng(seed).choice(x.shape[1], size=count, replace=False))
    y = x.copy()
    y[:, cols] *= np.float32(factor)
    return y, cols


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# -- the five workloads -------------------------------------------------------
def tiny():
    return {"W": normal((256, 256), 0), "A": normal((64, 256), 1)}


def sweep(dist: str, rows: int = 4096, cols: int = 4096):
    if dist == "normal":
        return normal((rows, cols), 2)
    if dist == "student_t3":
        return student_t((rows, cols), 3, 3.0)
    raise ValueError(dist)


def mxfp4_linear(M: int = 4096, K: int = 4096, N: int = 14336):
    x, cols = with_outlier_channels(normal((M, K), 4), 5)
    return {"X_bf16": to_bf16_bits(x), "outlier_cols": cols, "W": normal((N, K), 6, 0.02)}


RAZER_SPECIAL = (5.0, -5.0, 2.5, -2.5)


def razer_decode(M: int, N: int = 17408, K: int = 5120, with_weight: bool = True):
    seeds = {1: 8, 16: 9, 128: 10}
    a = to_bf16_bits(student_t((M, K), seeds.get(M, 100 + M), 4.0))
    out = {"A_bf16": a}
    if with_weight:
        out["W"] = normal((N, K), 7, 0.02)
    return out


PREFILL_N = (10240, 17408, 5120)


def prefill_act(M: int = 32768, K: int = 5120):
    return to_bf16_bits(student_t((M, K), 11, 4.0))


def prefill_weight(N: int, K: int = 5120):
    seed = {10240: 12, 17408: 13, 5120: 14}[N]
    return normal((N, K), seed, 0.02)
