"""GPU tests of bi_token_hash and bi_sample (through the C-ABI): the step after
the block.

Token hashes: the receipt page's two printed hashes, bit for bit, and the
oracle's BLAKE3 on lengths around block, chunk and tree boundaries.  Sampler:
greedy ids equal the oracle's exactly; seeded ids equal the oracle's wherever
the draw is not within a relative 1e-12 of a boundary between two candidates
(there either neighbour is correct, and the test checks the kernel's pick is
one of the two); every row's id is identical alone and batched.  The whole
step after a block (final RMSNorm, LM head over a 151936-token vocabulary,
sampling, hashing) runs on the GPU and its ids are checked against the oracle
sampler applied to the GPU's logits.
"""
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import sampling as S
from invariant_deterministic_amd import bi, synth
from tests.gpu_util import announce, assert_bitwise, bits, dev, device
from tests.util import assert_within_tolerance

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))


def hash_on_gpu(seqs):
    lens = np.array([len(s) for s in seqs], np.int32)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    flat = np.concatenate([np.asarray(s, np.int64) for s in seqs] + [np.zeros(1, np.int64)]).astype(np.uint32)
    ids = torch.from_numpy(flat.view(np.int32)).cuda()
    out = bi.token_hash(ids, torch.from_numpy(offs).cuda(), torch.from_numpy(lens).cuda())
    torch.cuda.synchronize()
    return [bytes(r) for r in out.cpu().numpy()]


def test_token_hash_receipt_page():
    device()
    rows = []
    with open(os.path.join(HERE, "golden", "receipt_token_hashes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            name, count, h, ids = (x.strip() for x in line.split("|"))
            rows.append((name, h, [int(t) for t in ids.split()]))
    announce("token hash, receipt page")
    got = hash_on_gpu([r[2] for r in rows])
    for (name, h, _), g in zip(rows, got):
        assert g.hex() == h, name


def test_token_hash_lengths_vs_oracle():
    device()
    rng = np.random.default_rng(8000)
    lens = [0, 1, 15, 16, 17, 255, 256, 257, 511, 512, 768, 1000, 1025, 4096, 4097, 20000, 65536]
    seqs = [rng.integers(0, 2 ** 32, size=n, dtype=np.uint64) for n in lens]
    announce("token hash lengths", lens)
    got = hash_on_gpu(seqs)
    for n, s, g in zip(lens, seqs, got):
        assert g == S.token_hash(s), f"length {n}"


def rand_logits(rng, rows, vocab, scale=3.0):
    return oracle.bf16_round(rng.standard_normal((rows, vocab)) * scale)


def run_sample(logit_bits, seeds, positions, hist=None, **kw):
    out = bi.sample(dev(logit_bits), torch.from_numpy(np.asarray(seeds, np.uint64).view(np.int64)).cuda(),
                    torch.from_numpy(np.asarray(positions, np.int64)).cuda(),
                    history=None if hist is None else torch.from_numpy(np.asarray(hist, np.int32)).cuda(), **kw)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_rows(got, logit_bits, seeds, positions, hist, params):
    near = 0
    for r in range(len(got)):
        h = () if hist is None else hist[r]
        want, det = S.sample_row(logit_bits[r], int(seeds[r]), int(positions[r]), params["temperature"],
                                 params["top_k"], params["top_p"], params["min_p"], h, params["repeat"],
                                 params["presence"], params["frequency"])
        if got[r] == want:
            continue
        assert det is not None, f"row {r}: greedy id {got[r]} != {want}"
        cs, tgt, ids = det["csum"], det["target"], list(det["ids"])
        i = ids.index(want)
        lo_b = cs[i - 1] if i > 0 else 0.0
        close = abs(tgt - lo_b) <= 1e-12 * cs[-1] or abs(tgt - cs[i]) <= 1e-12 * cs[-1]
        assert close and got[r] in ids[max(0, i - 1):i + 2], f"row {r}: id {got[r]} != {want}"
        near += 1
    return near


@pytest.mark.parametrize("vocab", [151936, 1000, 8])
def test_sample_greedy(vocab):
    device()
    rng = np.random.default_rng(8100 + vocab)
    rows = 48
    lg = rand_logits(rng, rows, vocab)
    lg[3, :] = lg[3, 0]                                   # all equal: id 0 without penalties
    lg[4, [5, vocab - 1]] = oracle.bf16_round(50.0)       # tie at the top: the lower id (5)
    hist = rng.integers(-3, vocab + 5, size=(rows, 64))   # includes ids outside the vocabulary
    prm = dict(temperature=0.0, top_k=1, top_p=1.0, min_p=0.0, repeat=1.3, presence=0.2, frequency=0.05)
    announce("sample greedy", vocab)
    seeds, pos = np.arange(rows) + 7, np.arange(rows) * 11
    got = run_sample(lg, seeds, pos, hist, **{k: prm[k] for k in ("temperature", "top_k", "top_p", "min_p", "repeat",
                                                                   "presence", "frequency")})
    check_rows(got, lg, seeds, pos, hist, prm)
    got0 = run_sample(lg, seeds, pos, None, temperature=0.0)
    assert np.array_equal(got0, np.argmax(oracle.bf16_decode(lg), axis=1))
    assert got0[3] == 0 and got0[4] == 5


@pytest.mark.parametrize("vocab,top_k,top_p,min_p,T", [(151936, 50, 0.95, 0.05, 0.8), (151936, 1024, 1.0, 0.0, 1.0),
                                                       (32000, 7, 0.5, 0.0, 1.5), (16, 50, 0.9, 0.01, 0.7)])
def test_sample_seeded_vs_oracle(vocab, top_k, top_p, min_p, T):
    device()
    rng = np.random.default_rng(8200 + top_k)
    rows = 96
    lg = rand_logits(rng, rows, vocab, 2.0)
    hist = rng.integers(0, vocab, size=(rows, 64))
    prm = dict(temperature=T, top_k=top_k, top_p=top_p, min_p=min_p, repeat=1.1, presence=0.1, frequency=0.05)
    seeds = rng.integers(0, 2 ** 63, size=rows, dtype=np.uint64) * 2 + 1
    pos = rng.integers(0, 100000, size=rows)
    announce("sample seeded", vocab, top_k, top_p, min_p, T)
    got = run_sample(lg, seeds, pos, hist, **prm)
    near = check_rows(got, lg, seeds, pos, hist, prm)
    print(f"  rows {rows}, draws within 1e-12 of a boundary: {near}")


def test_sample_batch_invariance():
    device()
    rng = np.random.default_rng(8300)
    rows, vocab = 40, 151936
    lg = rand_logits(rng, rows, vocab)
    hist = rng.integers(0, vocab, size=(rows, 32))
    seeds = rng.integers(0, 2 ** 62, size=rows, dtype=np.uint64)
    pos = rng.integers(0, 5000, size=rows)
    prm = dict(temperature=0.9, top_k=64, top_p=0.9, min_p=0.02, repeat=1.1)
    alone = [run_sample(lg[r:r + 1], seeds[r:r + 1], pos[r:r + 1], hist[r:r + 1], **prm)[0] for r in range(rows)]
    for B in (2, 17, 40):
        idx = rng.choice(rows, size=B, replace=False)
        announce("sample batch", B)
        got = run_sample(lg[idx], seeds[idx], pos[idx], hist[idx], **prm)
        assert_bitwise(got, np.array(alone)[idx], f"batch {B}")


def test_step_after_block():
    """Final RMSNorm, LM head (vocab 151936, hidden 2560), greedy and seeded sampling, token hash."""
    device()
    H, V, M = 2560, 151936, 64
    x = synth.normal_bf16(8400, (M, H))
    gamma = synth.normal_bf16(8401, (H,), 0.02, 1.0)
    w = synth.normal_bf16_device(8402, (V, H), 0.02)
    announce("step after block", M, V, H)
    n = bi.rmsnorm(dev(x), dev(gamma), 1e-6)
    logits = bi.gemm(n, w)
    lg = bits(logits)
    # final norm and LM-head logits against the oracle, per element, on sampled rows (the
    # whole vocabulary, in slices of the weight)
    nb = bits(n)
    assert_within_tolerance(nb, oracle.rmsnorm(x, gamma, 1e-6), "final RMSNorm")
    rows = np.array([0, 17, 42, M - 1])
    for c0 in range(0, V, 16384):
        wc = bits(w[c0:c0 + 16384])
        assert_within_tolerance(lg[rows, c0:c0 + len(wc)], oracle.gemm(nb[rows], wc), f"LM head logits {c0}..")
    seeds = np.arange(M, dtype=np.uint64) + 99
    pos = np.arange(M) + 4000
    prm = dict(temperature=0.8, top_k=50, top_p=0.95, min_p=0.05, repeat=1.0, presence=0.0, frequency=0.0)
    got = run_sample(lg, seeds, pos, None, **prm)
    check_rows(got, lg, seeds, pos, None, prm)
    greedy = run_sample(lg, seeds, pos, None, temperature=0.0)
    assert np.array_equal(greedy, np.argmax(oracle.bf16_decode(lg), axis=1))
    h = hash_on_gpu([got.astype(np.int64), greedy.astype(np.int64)])
    assert h[0] == S.token_hash(got) and h[1] == S.token_hash(greedy)
    # a row's logits and ids do not depend on the other rows
    half = bits(bi.gemm(bi.rmsnorm(dev(x[M // 2:]), dev(gamma), 1e-6), w))
    assert_bitwise(half, lg[M // 2:], "LM head rows alone")
