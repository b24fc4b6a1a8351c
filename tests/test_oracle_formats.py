"""Pins for the oracle's number formats: IEEE round-to-nearest-even into bf16.

bf16 is IEEE-754 binary32 with the low 16 mantissa bits dropped, so torch's
float32 -> bfloat16 conversion (round to nearest even) is an independent
library routine for every value that is itself a float32.  Values needing more
than 24 bits check that the oracle rounds float64 in one step, not via float32.
"""
import numpy as np
import pytest
import torch

from oracle import bf16_decode, bf16_round, f16_decode


def torch_bf16_bits(x32):
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_decode_known_patterns():
    assert bf16_decode(np.uint16(0x3F80)) == 1.0
    assert bf16_decode(np.uint16(0xC000)) == -2.0
    assert bf16_decode(np.uint16(0x0001)) == 2.0 ** -133
    assert bf16_decode(np.uint16(0x7F7F)) == (2 - 2 ** -7) * 2.0 ** 127
    assert f16_decode(np.uint16(0x3C00)) == 1.0
    assert f16_decode(np.uint16(0x0001)) == 2.0 ** -24
    assert f16_decode(np.uint16(0xC500)) == -5.0


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80),
    (1.0 + 2 ** -8, 0x3F80),            # tie, even mantissa below wins
    (1.0 + 3 * 2 ** -8, 0x3F82),        # tie, rounds up to the even mantissa
    (1.0 + 2 ** -8 + 2 ** -30, 0x3F81),  # just above the tie: up (a float32 detour would tie and go down)
    (-(1.0 + 2 ** -8 + 2 ** -30), 0xBF81),
    (0.0, 0x0000),
    (-0.0, 0x8000),
    (2.0 ** -133, 0x0001),              # smallest subnormal
    (2.0 ** -134, 0x0000),              # tie between 0 and 2^-133: to even (0)
    (1.5 * 2.0 ** -134, 0x0001),
    (3 * 2.0 ** -134, 0x0002),          # tie between 1 and 2 quanta: to even
    ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),
    ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),  # tie at the top: to even = infinity
    ((2 - 2 ** -7 + 2 ** -10) * 2.0 ** 127, 0x7F7F),
    (1e300, 0x7F80),
    (-1e300, 0xFF80),
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
])
def test_round_special_values(x, bits):
    assert int(bf16_round(np.float64(x))) == bits


def test_round_nan_stays_nan():
    b = int(bf16_round(np.float64("nan")))
    assert (b & 0x7F80) == 0x7F80 and (b & 0x7F) != 0


def test_round_matches_torch_on_float32_values():
    rng = np.random.default_rng(7)
    parts = [
        rng.standard_normal(200_000).astype(np.float32),
        (rng.standard_normal(50_000) * 1e-38).astype(np.float32),   # subnormal range
        (rng.standard_normal(50_000) * 1e37).astype(np.float32),
        rng.integers(-70000, 70000, 50_000).astype(np.float32),
    ]
    # exact ties: bf16 values plus half a bf16 ulp
    base = torch_bf16_bits(rng.standard_normal(50_000).astype(np.float32)).astype(np.uint32) << 16
    ties = (base | 0x8000).view(np.float32)
    parts.append(ties)
    x32 = np.concatenate(parts)
    x32 = x32[np.isfinite(x32)]
    np.testing.assert_array_equal(bf16_round(x32.astype(np.float64)), torch_bf16_bits(x32))


def test_roundtrip_every_finite_pattern():
    pats = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    finite = (pats & 0x7F80) != 0x7F80
    pats = pats[finite]
    back = bf16_round(bf16_decode(pats))
    np.testing.assert_array_equal(back, pats)
