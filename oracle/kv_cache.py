"""CPU oracle for the quantised, paged KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the bench's
CPU-baseline leg use anything under ``oracle/``.  It shares no code, table or
helper with the HIP library.

The "Receipts" page ("What a receipt proves") names a quantised cache among
the load settings that change the bits, and batch-invariant kernels must keep
a request's bits independent of where its cache lives.  The pages give no
format; the plain reading used here:

* int8, symmetric, one float32 scale per (token, kv head): with a = max |x_d|
  over the head's D values (x the bf16 key or value),
  scale = a / 127 (float32 division), q_d = clamp(rint(x_d / scale), -127, 127)
  (float32 division, ties to even); a = 0 gives scale 0 and q = 0.
* the value attention sees is bf16(float32(q_d) * scale): a float32 product,
  then one round-to-nearest-even to bf16.
* pages of 64 tokens: logical position p of a sequence lives in physical row
  block_table[p // 64] * 64 + p % 64 of the pool.

Attention over the cache is the plain attention definition (bi_oracle) applied
to the dequantised values in logical order.

Parity status: pinned by closed forms (constant heads, values on the int8
grid, zero heads, the rounding of the division and of the product) and by the
quantisation error bound (tests/test_oracle_kv_cache.py).
"""
from __future__ import annotations

import numpy as np

from .bi_oracle import bf16_decode, bf16_round

PAGE = 64


def quantize(x_bits):
    """bf16 [..., D] -> (int8 [..., D], float32 scale [...])."""
    x = bf16_decode(x_bits).astype(np.float32)
    a = np.abs(x).max(axis=-1)
    scale = (a / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(scale[..., None] > 0, x / np.where(scale > 0, scale, np.float32(1))[..., None], np.float32(0))
    q = np.clip(np.rint(r.astype(np.float32)), -127, 127).astype(np.int8)
    return q, scale


def dequantize(q, scale):
    """int8 [..., D], float32 [...] -> bf16 bits: bf16(float32(q) * scale)."""
    prod = (q.astype(np.float32) * scale.astype(np.float32)[..., None]).astype(np.float32)
    return bf16_round(prod.astype(np.float64))


def gather(pool, block_table, length):
    """Rows of one sequence (logical positions 0..length-1) from a paged pool."""
    pos = np.arange(length)
    rows = np.asarray(block_table, np.int64)[pos // PAGE] * PAGE + pos % PAGE
    return pool[rows]
