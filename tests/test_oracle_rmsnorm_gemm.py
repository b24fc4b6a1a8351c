"""Pins for the oracle's RMSNorm, GEMM and int4 de-quantisation.

RMSNorm: closed forms (constant rows, zero rows), exact power-of-two
symmetries, and brute force in 60-digit decimal arithmetic.  GEMM: exact
integer products (int64 matmul, then one float32 -> bf16 rounding in torch),
identity weights, and brute force in exact rational arithmetic.  int4:
hand-decoded bytes and exact integer GEMMs.
"""
import decimal
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import (bf16_decode, dequant_int4_g32, gemm, gemm_w4, int4_codes, rmsnorm)
from invariant_deterministic_amd import synth
from tests.util import assert_correctly_rounded, bf16_value

ONE = 0x3F80


def bits_of(vals):
    return synth.to_bf16_bits(np.asarray(vals, np.float32))


# ----------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("c", [2.0, 0.5, -3.0, 0.125, 100.0, -0.25])
def test_rmsnorm_constant_row_is_unit(c):
    # c / sqrt(c^2 + 1e-6) differs from sign(c) by < 5e-5, below half a bf16
    # ulp under 1 (2^-9), so the result is exactly +-1.
    x = bits_of(np.full((3, 256), c))
    y = rmsnorm(x, synth.ones_bf16(256), 1e-6)
    assert np.all(y == (ONE if c > 0 else 0xBF80))


def test_rmsnorm_small_constant_sees_eps():
    # c = bf16(1e-4): c^2 ~ 1e-8 is comparable to eps = 1e-6, so eps matters.
    x = bits_of(np.full((1, 64), 1e-4))
    c = Fraction(float(bf16_value(x[0, 0])))
    eps = Fraction(float(np.float32(1e-6)))
    ctx = decimal.Context(prec=60)
    exact = float(ctx.divide(decimal.Decimal(c.numerator) / decimal.Decimal(c.denominator),
                             (decimal.Decimal((c * c + eps).numerator) /
                              decimal.Decimal((c * c + eps).denominator)).sqrt(ctx)))
    y = rmsnorm(x, synth.ones_bf16(64), 1e-6)
    assert 0.09 < exact < 0.11
    assert_correctly_rounded(y, np.full(y.shape, exact))


def test_rmsnorm_zero_row():
    y = rmsnorm(np.zeros((2, 128), np.uint16), synth.ones_bf16(128), 1e-6)
    assert np.all(y == 0)


def test_rmsnorm_symmetries():
    x = synth.normal_bf16(11, (5, 96))
    g = synth.normal_bf16(12, (96,), 0.02, 1.0)
    y = rmsnorm(x, g, 1e-6)
    # gain doubles -> output doubles exactly (power of two, no overflow)
    g2 = synth.to_bf16_bits(2 * bf16_value(g).astype(np.float32))
    np.testing.assert_array_equal(bf16_value(rmsnorm(x, g2, 1e-6)), 2 * bf16_value(y))
    # sign flip of x flips the output
    np.testing.assert_array_equal(rmsnorm(x ^ np.uint16(0x8000), g, 1e-6) ^ np.uint16(0x8000), y)
    # with eps = 0, scaling x by 2 changes nothing (sqrt of 4s is exactly 2 sqrt(s))
    x2 = synth.to_bf16_bits(2 * bf16_value(x).astype(np.float32))
    np.testing.assert_array_equal(rmsnorm(x2, g, 0.0), rmsnorm(x, g, 0.0))
    # rows are independent: a row alone gives the same bits as in the batch
    for r in range(5):
        np.testing.assert_array_equal(rmsnorm(x[r:r + 1], g, 1e-6)[0], y[r])


def test_rmsnorm_brute_force_decimal():
    ctx = decimal.Context(prec=60)
    D = decimal.Decimal
    x = synth.normal_bf16(13, (4, 7))
    g = synth.normal_bf16(14, (7,), 0.5, 1.0)
    xv = bf16_value(x)
    gv = bf16_value(g)
    eps = D(float(np.float32(1e-6)))
    exact = np.empty(xv.shape)
    for r in range(xv.shape[0]):
        ss = sum((D(float(v)) * D(float(v)) for v in xv[r]), D(0))
        inv = D(1) / ctx.sqrt(ss / D(xv.shape[1]) + eps)
        for j in range(xv.shape[1]):
            exact[r, j] = float(D(float(xv[r, j])) * inv * D(float(gv[j])))
    assert_correctly_rounded(rmsnorm(x, g, 1e-6), exact)


# -------------------------------------------------------------------- GEMM
def torch_round_exact_ints(c_int):
    assert np.abs(c_int).max() < 2 ** 24
    return synth.to_bf16_bits(c_int.astype(np.float32))


@pytest.mark.parametrize("m,n,k", [(5, 7, 64), (3, 9, 4096), (17, 33, 250)])
def test_gemm_small_integers_exact(m, n, k):
    a = synth.small_int_bf16(21, (m, k))
    w = synth.small_int_bf16(22, (n, k))
    ai = bf16_value(a).astype(np.int64)
    wi = bf16_value(w).astype(np.int64)
    np.testing.assert_array_equal(gemm(a, w), torch_round_exact_ints(ai @ wi.T))


def test_gemm_identity_weight():
    a = synth.normal_bf16(23, (6, 40))
    eye = synth.to_bf16_bits(np.eye(40, dtype=np.float32))
    np.testing.assert_array_equal(gemm(a, eye), a)


def test_gemm_brute_force_rational():
    a = synth.normal_bf16(24, (3, 19))
    w = synth.normal_bf16(25, (4, 19))
    av, wv = bf16_value(a), bf16_value(w)
    exact = np.empty((3, 4))
    for i in range(3):
        for j in range(4):
            exact[i, j] = float(sum((Fraction(float(av[i, k])) * Fraction(float(wv[j, k]))
                                     for k in range(19)), Fraction(0)))
    assert_correctly_rounded(gemm(a, w), exact)


def test_gemm_rows_independent():
    a = synth.normal_bf16(26, (9, 128))
    w = synth.normal_bf16(27, (16, 128))
    c = gemm(a, w)
    perm = np.random.default_rng(0).permutation(9)
    np.testing.assert_array_equal(gemm(a[perm], w), c[perm])


# -------------------------------------------------------------------- int4
def test_int4_nibble_order_and_sign():
    wq = np.array([[0x9F, 0x78, 0x00, 0x81]], dtype=np.uint8)
    # byte 0x9F: low nibble F = -1 (element 0), high nibble 9 = -7 (element 1)
    # byte 0x78: low 8 = -8, high 7 = 7; byte 0x81: low 1, high 8 = -8
    np.testing.assert_array_equal(int4_codes(wq), [[-1, -7, -8, 7, 0, 0, 1, -8]])


def test_int4_dequant_scales_per_group():
    k = 64
    codes = (np.arange(k) % 16) - 8
    nib = (codes & 0xF).astype(np.uint8)
    wq = (nib[0::2] | (nib[1::2] << 4))[None, :]
    # fp16 1.0 for group 0, fp16 0.5 for group 1
    ws = np.array([[0x3C00, 0x3800]], dtype=np.uint16)
    w = bf16_value(dequant_int4_g32(wq, ws))[0]
    np.testing.assert_array_equal(w[:32], codes[:32].astype(np.float64))
    np.testing.assert_array_equal(w[32:], codes[32:] * 0.5)


def test_int4_dequant_rounds_product_to_bf16():
    # scale 1 + 2^-10 (fp16 0x3C01): q * s needs more than 8 significant bits
    codes = np.array([7, 3, -5, 1] * 8)
    nib = (codes & 0xF).astype(np.uint8)
    wq = (nib[0::2] | (nib[1::2] << 4))[None, :]
    ws = np.array([[0x3C01]], dtype=np.uint16)
    s = 1 + 2 ** -10
    assert_correctly_rounded(dequant_int4_g32(wq, ws)[0], codes * s)


def test_gemm_w4_exact_with_unit_scales():
    n, k, m = 12, 256, 5
    rng = np.random.default_rng(31)
    codes = rng.integers(-8, 8, size=(n, k))
    nib = (codes & 0xF).astype(np.uint8)
    wq = nib[:, 0::2] | (nib[:, 1::2] << 4)
    ws = np.full((n, k // 32), 0x3C00, np.uint16)
    a = synth.small_int_bf16(32, (m, k))
    exact = bf16_value(a).astype(np.int64) @ codes.T
    np.testing.assert_array_equal(gemm_w4(a, wq, ws), torch_round_exact_ints(exact))


def test_synth_quantizer_roundtrip_within_half_step():
    wq, ws = synth.quantize_int4_g32(41, 8, 64, 0.02)
    rng = np.random.default_rng(41)
    w = rng.standard_normal(size=(8, 64), dtype=np.float32) * np.float32(0.02)
    deq = bf16_value(dequant_int4_g32(wq, ws))
    s = np.repeat(ws.view(np.float16).astype(np.float64), 32, axis=1)
    # half a quantisation step plus the bf16 rounding of q*s (|q*s| <= 8s)
    assert np.all(np.abs(deq - w) <= 0.5 * s + 8 * s * 2 ** -9 + 1e-9)
