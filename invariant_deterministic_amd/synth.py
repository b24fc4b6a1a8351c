"""Seeded synthetic inputs shared by the tests, the bench and the CPU checker.

This module draws random inputs and stores them in the formats the library
consumes (bf16 bit patterns, packed int4 with fp16 group scales, int32/int64
metadata).  It holds none of the arithmetic of the forward path itself: no
normalisation, no products, no softmax.  Every array it returns is host memory
(numpy); moving it to the device is the caller's business.

Recipe: ``numpy.random.default_rng(seed)`` standard normal draws in float32,
times sigma, rounded once to bf16 (round-to-nearest-even, done by torch's
float32 -> bfloat16 conversion).  Seeds follow ``100 * config + tensor index``.
"""
from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "to_bf16_bits",
    "normal_bf16",
    "small_int_bf16",
    "ones_bf16",
    "quantize_int4_g32",
    "uniform_ints",
    "normal_bf16_device",
]


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    """Round a float32 array to bf16 (RNE) and return the raw uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(seed: int, shape, sigma: float = 1.0, mean: float = 0.0) -> np.ndarray:
    """bf16 bits of mean + sigma * N(0, 1) drawn from default_rng(seed)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x = x * np.float32(sigma) + np.float32(mean)
    return to_bf16_bits(x)


def small_int_bf16(seed: int, shape, lo: int = -3, hi: int = 3) -> np.ndarray:
    """bf16 bits of integers drawn uniformly from [lo, hi] (exactly representable)."""
    rng = np.random.default_rng(seed)
    x = rng.integers(lo, hi + 1, size=shape).astype(np.float32)
    return to_bf16_bits(x)


def ones_bf16(shape) -> np.ndarray:
    return np.full(shape, 0x3F80, dtype=np.uint16)


def quantize_int4_g32(seed: int, n: int, k: int, sigma: float = 0.02):
    """Random weights W[n, k] ~ N(0, sigma) stored as symmetric int4, group 32 along k.

    Returns ``(wq, ws)``: ``wq`` uint8 [n, k/2] with element 2i in the low nibble
    and element 2i+1 in the high nibble of byte i (two's complement, range
    [-8, 7]); ``ws`` uint16 [n, k/32] holding the fp16 bit pattern of each
    group's scale.  The scale is max|w|/7 of the group rounded to fp16, and the
    code is clamp(round_half_even(w / scale), -8, 7).  Only ``wq`` and ``ws``
    define the weight: both the library and the checker decode these bytes.
    """
    if k % 32:
        raise ValueError("k must be a multiple of 32")
    rng = np.random.default_rng(seed)
    w = rng.standard_normal(size=(n, k), dtype=np.float32) * np.float32(sigma)
    g = w.reshape(n, k // 32, 32)
    amax = np.abs(g).max(axis=2)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s16 = np.where(s16 == 0, np.float16(1.0), s16)
    q = np.rint(g / s16.astype(np.float32)[:, :, None])
    q = np.clip(q, -8, 7).astype(np.int8).reshape(n, k)
    nib = (q.astype(np.int16) & 0xF).astype(np.uint8)
    wq = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    ws = s16.view(np.uint16).copy()
    return np.ascontiguousarray(wq), np.ascontiguousarray(ws)


def uniform_ints(seed: int, count: int, lo: int, hi: int) -> np.ndarray:
    """``count`` integers drawn uniformly from [lo, hi] inclusive (int64)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=count).astype(np.int64)


def normal_bf16_device(seed: int, shape, sigma: float = 1.0, device="cuda"):
    """Large seeded N(0, sigma) bf16 tensors drawn on the device (torch's Philox
    generator), for inputs too big to draw on the host (KV caches).  The same
    seed gives the same tensor on every run; tests copy the parts the checker
    needs back to the host."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)
