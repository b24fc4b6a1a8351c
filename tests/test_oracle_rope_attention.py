"""Pins for the oracle's rotary embedding, attention and elementwise steps.

RoPE: position 0 is the identity; a single pair is multiplication by a
complex exponential (numpy complex arithmetic as the independent routine);
the frequency of pair i is theta^(-2i/D).  Attention: one visible key gives
exactly v; identical keys give the plain mean; two keys give the logistic
function (scipy.special.expit); the GQA head map, the causal mask and absolute
positions are pinned with constructed data; tiny cases are brute forced in
pure Python.  Elementwise: torch's bf16 add and scipy's expit.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import (attention, attention_weights, decode_attention, residual_add,
                    rope, swiglu)
from invariant_deterministic_amd import synth
from tests.util import assert_correctly_rounded, bf16_value


# -------------------------------------------------------------------- RoPE
def test_rope_position_zero_is_identity():
    x = synth.normal_bf16(51, (3, 4, 128))
    np.testing.assert_array_equal(rope(x, [0, 0, 0], 1e6), x)


@pytest.mark.parametrize("p", [1, 2, 7, 100, 4095])
def test_rope_single_pair_is_complex_rotation(p):
    # D = 2: one pair, frequency theta^0 = 1, so the pair turns by p radians.
    x = synth.normal_bf16(52, (1, 3, 2))
    xv = bf16_value(x)
    z = (xv[..., 0] + 1j * xv[..., 1]) * np.exp(1j * p)
    y = rope(x, [p], 1e6)
    assert_correctly_rounded(y[..., 0], z.real, rel_slack=1e-9, abs_slack=1e-12)
    assert_correctly_rounded(y[..., 1], z.imag, rel_slack=1e-9, abs_slack=1e-12)


def test_rope_second_pair_frequency():
    # D = 4, theta = 100: pair 1 = (x1, x3) turns at 100^(-2/4) = 0.1 rad per position.
    x = synth.normal_bf16(53, (5, 1, 4))
    pos = np.array([0, 1, 3, 10, 31])
    xv = bf16_value(x)
    z = (xv[:, 0, 1] + 1j * xv[:, 0, 3]) * np.exp(1j * 0.1 * pos)
    y = rope(x, pos, 100.0)
    assert_correctly_rounded(y[:, 0, 1], z.real, rel_slack=1e-9, abs_slack=1e-12)
    assert_correctly_rounded(y[:, 0, 3], z.imag, rel_slack=1e-9, abs_slack=1e-12)
    z0 = (xv[:, 0, 0] + 1j * xv[:, 0, 2]) * np.exp(1j * 1.0 * pos)
    assert_correctly_rounded(y[:, 0, 0], z0.real, rel_slack=1e-9, abs_slack=1e-12)


def test_rope_relative_position_property():
    q = synth.normal_bf16(54, (1, 1, 64))
    k = synth.normal_bf16(55, (1, 1, 64))
    dots = []
    for shift in (0, 17, 300):
        a = bf16_value(rope(q, [40 + shift], 1e4))
        b = bf16_value(rope(k, [12 + shift], 1e4))
        dots.append(float((a * b).sum()))
    # equal up to the bf16 rounding of the rotated vectors
    assert max(dots) - min(dots) < 0.2


# --------------------------------------------------------------- attention
SCALE = 1.0 / math.sqrt(64)


def test_single_key_returns_v():
    q = synth.normal_bf16(61, (1, 4, 64))
    k = synth.normal_bf16(62, (1, 4, 64))
    v = synth.normal_bf16(63, (1, 4, 64))
    np.testing.assert_array_equal(attention(q, k, v, [0], SCALE), v)


def test_first_query_sees_only_first_key():
    q = synth.normal_bf16(64, (6, 8, 64))
    k = synth.normal_bf16(65, (6, 2, 64))
    v = synth.normal_bf16(66, (6, 2, 64))
    o = attention(q, k, v, np.arange(6), SCALE)
    for h in range(8):
        np.testing.assert_array_equal(o[0, h], v[0, h // 4])


def test_decode_single_key():
    q = synth.normal_bf16(67, (32, 128))
    k = synth.normal_bf16(68, (1, 8, 128))
    v = synth.normal_bf16(69, (1, 8, 128))
    o = decode_attention(q, k, v, 1 / math.sqrt(128))
    for h in range(32):
        np.testing.assert_array_equal(o[h], v[0, h // 4])


def test_identical_keys_give_mean():
    L = 37
    q = synth.normal_bf16(70, (1, 2, 64))
    k1 = synth.normal_bf16(71, (1, 1, 64))
    k = np.repeat(k1, L, axis=0)
    v = synth.normal_bf16(72, (L, 1, 64))
    o = attention(q, k, v, [L - 1], SCALE)
    mean = bf16_value(v)[:, 0, :].mean(axis=0)
    for h in range(2):
        assert_correctly_rounded(o[0, h], mean, rel_slack=1e-9, abs_slack=1e-15)


def test_two_keys_logistic():
    # q = a e0, k0 = e0, k1 = 0: logits (a*scale, 0), weights expit(+-a*scale).
    D = 64
    for a in (0.5, 3.0, -7.25, 20.0):
        qf = np.zeros((1, 1, D), np.float32); qf[0, 0, 0] = a
        kf = np.zeros((2, 1, D), np.float32); kf[0, 0, 0] = 1.0
        q = synth.to_bf16_bits(qf); k = synth.to_bf16_bits(kf)
        v = synth.normal_bf16(73, (2, 1, D))
        vv = bf16_value(v)[:, 0, :]
        w0 = scipy.special.expit(a * SCALE)
        exact = w0 * vv[0] + (1 - w0) * vv[1]
        o = attention(q, k, v, [1], SCALE)
        assert_correctly_rounded(o[0, 0], exact, rel_slack=1e-9, abs_slack=1e-15)


def test_gqa_head_mapping():
    # kv head 0 carries v = 1, kv head 1 carries v = 2: q heads 0,1 -> 1; 2,3 -> 2
    L = 5
    q = synth.normal_bf16(74, (1, 4, 64))
    k = synth.normal_bf16(75, (L, 2, 64))
    vf = np.zeros((L, 2, 64), np.float32); vf[:, 0] = 1.0; vf[:, 1] = 2.0
    o = bf16_value(attention(q, k, synth.to_bf16_bits(vf), [L - 1], SCALE))
    assert np.all(o[0, :2] == 1.0) and np.all(o[0, 2:] == 2.0)


def test_future_keys_do_not_matter():
    T = 12
    q = synth.normal_bf16(76, (T, 4, 64))
    k = synth.normal_bf16(77, (T, 4, 64))
    v = synth.normal_bf16(78, (T, 4, 64))
    o = attention(q, k, v, np.arange(T), SCALE)
    k2, v2 = k.copy(), v.copy()
    k2[7:] = synth.normal_bf16(79, (T - 7, 4, 64))
    v2[7:] = synth.normal_bf16(80, (T - 7, 4, 64))
    o2 = attention(q, k2, v2, np.arange(T), SCALE)
    np.testing.assert_array_equal(o[:7], o2[:7])
    assert not np.array_equal(o[7:], o2[7:])


def test_chunked_queries_equal_whole():
    # positions are absolute: a chunk of queries over the same cache gives the same bits
    T = 40
    q = synth.normal_bf16(81, (T, 4, 64))
    k = synth.normal_bf16(82, (T, 2, 64))
    v = synth.normal_bf16(83, (T, 2, 64))
    whole = attention(q, k, v, np.arange(T), SCALE)
    for start in (0, 9, 25):
        end = min(T, start + 11)
        part = attention(q[start:end], k[:end], v[:end], np.arange(start, end), SCALE)
        np.testing.assert_array_equal(part, whole[start:end])


def test_softmax_rows_sum_to_one_and_mask():
    T = 30
    q = bf16_value(synth.normal_bf16(84, (T, 4, 64)))
    k = bf16_value(synth.normal_bf16(85, (T, 2, 64)))
    p = attention_weights(q, k, np.arange(T), SCALE)
    np.testing.assert_allclose(p.sum(axis=2), 1.0, rtol=0, atol=1e-12)
    future = np.triu(np.ones((T, T), bool), 1)
    assert np.all(p[:, future] == 0.0)


def test_attention_brute_force_python():
    T, Hq, Hkv, D = 5, 2, 1, 8
    q = synth.normal_bf16(86, (T, Hq, D))
    k = synth.normal_bf16(87, (T, Hkv, D))
    v = synth.normal_bf16(88, (T, Hkv, D))
    qv, kv, vv = bf16_value(q).tolist(), bf16_value(k).tolist(), bf16_value(v).tolist()
    sc = 0.3
    exact = np.zeros((T, Hq, D))
    for t in range(T):
        for h in range(Hq):
            z = [math.fsum(qv[t][h][e] * kv[s][0][e] for e in range(D)) * sc for s in range(t + 1)]
            mx = max(z)
            w = [math.exp(zi - mx) for zi in z]
            tot = math.fsum(w)
            for e in range(D):
                exact[t, h, e] = math.fsum(w[s] * vv[s][0][e] for s in range(t + 1)) / tot
    assert_correctly_rounded(attention(q, k, v, np.arange(T), sc), exact, rel_slack=1e-9, abs_slack=1e-15)


# ------------------------------------------------------------- elementwise
def test_residual_add_matches_torch_bf16_add():
    # torch adds bf16 in float32 and rounds once; float32 has more than 2*8+2
    # bits, so that double rounding equals a single exact rounding.
    x = synth.normal_bf16(91, (64, 300))
    o = synth.normal_bf16(92, (64, 300), 0.3)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    to = torch.from_numpy(o.view(np.int16)).view(torch.bfloat16)
    ref = (tx + to).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(residual_add(x, o), ref)


def test_swiglu_against_expit():
    g = synth.normal_bf16(93, (10, 77), 3.0)
    u = synth.normal_bf16(94, (10, 77))
    gv, uv = bf16_value(g), bf16_value(u)
    exact = gv * scipy.special.expit(gv) * uv
    assert_correctly_rounded(swiglu(g, u), exact, rel_slack=1e-12, abs_slack=1e-300)


def test_swiglu_zero_gate():
    u = synth.normal_bf16(95, (4, 16))
    out = swiglu(np.zeros((4, 16), np.uint16), u)
    assert np.all(bf16_value(out) == 0.0)
