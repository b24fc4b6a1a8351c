"""CPU pins of oracle/kv_cache.py: int8 per-(token, head) quantisation, its
dequantised values, and paged addressing."""
import numpy as np

import oracle
from oracle import kv_cache as KV


def _bits(x):
    return oracle.bf16_round(np.asarray(x, np.float64))


def test_constant_head_quantises_to_127():
    x = _bits(np.full((3, 2, 64), -0.75))
    q, s = KV.quantize(x)
    assert np.all(q == -127) and np.all(s == np.float32(0.75) / np.float32(127))
    # dequantised: bf16(float32(-127) * float32(0.75 / 127)) is -0.75 again
    assert np.all(KV.dequantize(q, s) == x)


def test_zero_head():
    q, s = KV.quantize(np.zeros((2, 1, 128), np.uint16))
    assert np.all(q == 0) and np.all(s == 0)
    assert np.all(KV.dequantize(q, s) == 0)


def test_values_on_the_grid_are_exact():
    """x = k * 2^-7 with max |k| = 127: scale = 127 * 2^-7 / 127 = 2^-7 exactly, q = k."""
    rng = np.random.default_rng(1)
    k = rng.integers(-127, 128, size=(50, 64))
    k[:, 0] = 127
    x = _bits(k * 2.0 ** -7)
    q, s = KV.quantize(x)
    assert np.all(s == np.float32(2.0 ** -7))
    assert np.array_equal(q.astype(np.int64), k)
    assert np.array_equal(KV.dequantize(q, s), x)


def test_rounding_ties_to_even_and_clamp():
    # a = 127: scale 1; x = 2.5 -> 2, 3.5 -> 4, -2.5 -> -2
    x = _bits([127.0, 2.5, 3.5, -2.5, 0.5, 1.5] + [0.0] * 58)
    q, s = KV.quantize(x)
    assert s == 1.0
    assert list(q[:6]) == [127, 2, 4, -2, 0, 2]


def test_error_bound():
    """|x - dequant| <= scale / 2 (+ the bf16 rounding of the product)."""
    rng = np.random.default_rng(2)
    x = _bits(rng.standard_normal((200, 8, 128)) * np.exp(rng.uniform(-8, 8, (200, 8, 1))))
    q, s = KV.quantize(x)
    xd = oracle.bf16_decode(x)
    dq = oracle.bf16_decode(KV.dequantize(q, s))
    bound = s[..., None].astype(np.float64) * 0.5 * (1 + 1e-6) + np.abs(dq) * 2.0 ** -8
    assert np.all(np.abs(xd - dq) <= bound)
    assert np.all(np.abs(q.astype(np.int64)) <= 127)


def test_paged_gather():
    pool = np.arange(5 * KV.PAGE)[:, None]
    table = [3, 0, 4]
    g = KV.gather(pool, table, 150)
    assert g[0, 0] == 3 * 64 and g[63, 0] == 3 * 64 + 63 and g[64, 0] == 0 and g[128, 0] == 4 * 64
    assert g.shape == (150, 1)
