"""CPU pins of oracle/sampling.py: BLAKE3 token hashes, Philox4x64-10 draws and
the seeded sampler.

Pins: the two token hashes printed by the "Receipts" page (tests/golden);
numpy's own Philox generator for the random words; closed forms for each
sampler step (penalties, greedy, top-k = 1, min-p, top-p) and a chi-square
test of the sampled distribution against the tempered softmax.
"""
import os

import numpy as np
import pytest

import oracle
from oracle import sampling as S

HERE = os.path.dirname(os.path.abspath(__file__))


def golden_receipt():
    rows = []
    with open(os.path.join(HERE, "golden", "receipt_token_hashes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, count, h, ids = (x.strip() for x in line.split("|"))
            rows.append((name, int(count), h, [int(t) for t in ids.split()]))
    return rows


def test_token_hashes_match_the_receipt_page():
    rows = golden_receipt()
    assert len(rows) == 2
    for name, count, h, ids in rows:
        assert len(ids) == count
        assert S.token_hash(ids).hex() == h, name


def test_token_hash_is_over_little_endian_u32():
    ids = [1, 2, 0x01020304]
    assert S.token_hash(ids) == S.blake3(b"\x01\x00\x00\x00\x02\x00\x00\x00\x04\x03\x02\x01")
    # one changed id changes the hash; so does the order
    rows = golden_receipt()
    ids = list(rows[1][3])
    assert S.token_hash(ids[:-1] + [ids[-1] + 1]).hex() != rows[1][2]
    assert S.token_hash(ids[::-1]).hex() != rows[1][2]


def test_blake3_structure():
    """Lengths around block and chunk boundaries give distinct digests of 32 bytes; the
    tree (more than one chunk) is exercised; single-chunk digests are pinned above."""
    seen = set()
    for n in (0, 1, 63, 64, 65, 1023, 1024, 1025, 2048, 2049, 3072, 5121):
        d = S.blake3(bytes(i % 251 for i in range(n)))
        assert len(d) == 32
        seen.add(d)
    assert len(seen) == 12


def test_philox_matches_numpy():
    """numpy's Philox (4 x 64, 10 rounds) increments its counter before the first block."""
    for ctr, key in ((0, (0, 0)), (5, (7, 9)), (2 ** 40 + 3, (0xDEADBEEF12345678, 1)), (2 ** 64 - 1, (3, 0))):
        bg = np.random.Philox(counter=(ctr - 1) % 2 ** 256, key=key[0] + (key[1] << 64))
        want = [int(x) for x in bg.random_raw(4)]
        c = [ctr & (2 ** 64 - 1), ctr >> 64, 0, 0]
        assert S.philox4x64_10(c, key) == want


def test_uniform_draws():
    u = np.array([S.uniform(42, p) for p in range(4000)])
    assert np.all((u >= 0) & (u < 1))
    assert abs(u.mean() - 0.5) < 0.02 and abs(u.var() - 1 / 12) < 0.01
    assert S.uniform(42, 7) != S.uniform(43, 7)


def _bits(x):
    return oracle.bf16_round(np.asarray(x, np.float64))


def test_penalties_closed_form():
    l = _bits([2.0, -2.0, 1.5, 0.5])
    p = S.penalised_logits(l, [0, 1, 1, -1], repeat=2.0)
    assert list(p) == [1.0, -4.0, 1.5, 0.5]
    p = S.penalised_logits(l, [2, 2, 2, 3], presence=0.5, frequency=0.25)
    assert list(p) == [2.0, -2.0, 1.5 - (0.5 + 3 * 0.25), 0.5 - 0.75]


def test_greedy_and_top_k_one():
    rng = np.random.default_rng(5)
    for _ in range(20):
        l = _bits(rng.standard_normal(300))
        want = int(np.argmax(oracle.bf16_decode(l)))
        assert S.sample_row(l, 1, 2, 0.0, 50, 0.9, 0.0)[0] == want
        assert S.sample_row(l, 1, 2, 0.7, 1, 1.0, 0.0)[0] == want
    l = _bits([1.0, 3.0, 3.0, 0.0])
    assert S.sample_row(l, 1, 0, 0.0, 4, 1.0, 0.0)[0] == 1          # lowest id on ties


def test_min_p_and_top_p_closed_forms():
    # T = 1, logits 0, -1, -2, -3: weights 1, e^-1, e^-2, e^-3
    l = _bits([0.0, -1.0, -2.0, -3.0])
    _, d = S.sample_row(l, 3, 9, 1.0, 4, 1.0, 0.3)                    # e^-1 = 0.37 kept, e^-2 = 0.14 not
    assert list(d["ids"]) == [0, 1]
    eq = _bits([1.0, 1.0, 1.0, 1.0])
    _, d = S.sample_row(eq, 3, 9, 1.0, 4, 0.5, 0.0)
    assert list(d["ids"]) == [0, 1]                                   # 2/4 reaches 0.5
    _, d = S.sample_row(eq, 3, 9, 1.0, 4, 0.51, 0.0)
    assert list(d["ids"]) == [0, 1, 2]
    _, d = S.sample_row(eq, 3, 9, 1.0, 2, 1.0, 0.0)
    assert list(d["ids"]) == [0, 1]                                   # top-k keeps the lowest ids on ties


def test_sampled_distribution_matches_tempered_softmax():
    """Chi-square over 20000 positions: frequencies follow exp(l / T) renormalised over the kept set."""
    rng = np.random.default_rng(11)
    l = _bits(rng.standard_normal(12) * 1.5)
    T, n = 0.8, 20000
    counts = np.zeros(12)
    for pos in range(n):
        counts[S.sample_row(l, 1234, pos, T, 12, 1.0, 0.0)[0]] += 1
    z = oracle.bf16_decode(l).astype(np.float32).astype(np.float64)
    p = np.exp((z - z.max()) / np.float64(np.float32(T)))
    p /= p.sum()
    chi2 = float(((counts - n * p) ** 2 / (n * p)).sum())
    assert chi2 < 45.0        # 11 degrees of freedom: P(chi2 > 45) ~ 5e-6
