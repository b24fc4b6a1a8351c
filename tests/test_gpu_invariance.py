"""Batch invariance of the standalone kernels, counted by the invariance harness:
every request's output bits across lone runs, batches of many sizes, positions
and orders, and repeats ("Receipts", "Same input, same output": repeated runs,
count the distinct answers; M-0002 `technical`: a fixed reduction order per
element whatever the batch size).  Each report prints the rows compared, the
percentage identical and the largest number of distinct outputs of a request.

- bf16 GEMM, K = N = 4096: row i of C at M in {1, 7, 64, 288, 385, 513, 4096}, identity,
  reversed and random orders (64 rows also alone, 10 times for 8 of them).
- RMSNorm at hidden 2560 and 4096: rows alone and in batches up to 4096.
- Decode attention, 32 / 8 heads x 128, KV lengths ~ U{1..32768}: 64 requests alone
  (10 times each) and in batches of 1..64, random, reversed and rotated orders,
  with the grid sized for a longer request than any in the batch.
"""
import math

import numpy as np
import pytest
import torch

from invariant_deterministic_amd import bi, harness, synth
from tests.gpu_util import announce, bits, dev, device

pytestmark = pytest.mark.gpu


def test_gemm_rows_invariance():
    device()
    A = dev(synth.normal_bf16(201, (4096, 4096)))
    W = dev(synth.normal_bf16(202, (4096, 4096)))

    def backend(reqs, variant):
        idx = torch.tensor(reqs, dtype=torch.int64, device="cuda")
        c = bits(bi.gemm(A.index_select(0, idx).contiguous(), W))
        return [c[j:j + 1] for j in range(len(reqs))]

    rng = np.random.default_rng(203)
    every = tuple(range(4096))
    calls = [harness.Call(every, None, "M=4096 identity"), harness.Call(every[::-1], None, "M=4096 reversed"),
             harness.Call(tuple(int(i) for i in rng.permutation(4096)), None, "M=4096 random")]
    for M in (1, 7, 64, 288, 385, 513):
        for name in ("random", "random again"):
            calls.append(harness.Call(tuple(int(i) for i in rng.choice(4096, M, replace=False)), None, f"M={M} {name}"))
    sample = [int(i) for i in rng.choice(4096, 64, replace=False)]
    calls += [harness.Call((i,), None, f"alone row {i}") for i in sample]
    calls += [harness.Call((i,), None, f"alone row {i} rep {r}") for r in range(1, 10) for i in sample[:8]]
    rep = harness.run(backend, calls, log=lambda m: None if m.startswith("alone") else announce("gemm", m))
    print("GEMM rows:", rep.summary())
    assert rep.invariant and rep.identical_pct == 100.0, rep.summary()
    assert len(rep.distinct) == 4096 and all(rep.observations[i] >= 12 for i in sample[:8])


@pytest.mark.parametrize("hidden", [2560, 4096])
def test_rmsnorm_rows_invariance(hidden):
    device()
    x = dev(synth.normal_bf16(60 + hidden, (4096, hidden)))
    g = dev(synth.normal_bf16(61 + hidden, (hidden,), 0.02, 1.0))

    def backend(reqs, variant):
        idx = torch.tensor(reqs, dtype=torch.int64, device="cuda")
        y = bits(bi.rmsnorm(x.index_select(0, idx).contiguous(), g, 1e-6))
        return [y[j:j + 1] for j in range(len(reqs))]

    calls = [harness.Call(tuple(range(4096)), None, "all rows")]
    calls += harness.plan(range(4096), [1, 7, 64, 513, 2049, 4096], repeats=0, batch_repeats=2, seed=hidden)
    calls += [harness.Call((i,), None, f"alone {i} rep {r}") for r in range(10) for i in (0, 1, 4095)]
    rep = harness.run(backend, calls)
    print(f"RMSNorm rows (hidden {hidden}):", rep.summary())
    assert rep.invariant and rep.identical_pct == 100.0, rep.summary()


def test_decode_requests_invariance():
    device()
    hq, hkv, d = 32, 8, 128
    lens = synth.uniform_ints(401, 64, 1, 32768)
    total = int(lens.sum())
    k = synth.normal_bf16_device(403, (total, hkv, d))
    v = synth.normal_bf16_device(404, (total, hkv, d))
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    q = dev(synth.normal_bf16(402, (64, hq * d)))
    offs_d = torch.from_numpy(offs).cuda()
    lens_d = torch.from_numpy(lens.astype(np.int32)).cuda()
    ncall = [0]

    def backend(reqs, variant):
        idx = torch.tensor(reqs, dtype=torch.int64, device="cuda")
        # grid sized for up to 2 units more than the batch needs, varying by call
        max_len = int(lens[list(reqs)].max()) + 256 * (ncall[0] % 3)
        ncall[0] += 1
        o = bi.attn_decode(q.index_select(0, idx).contiguous(), k, v, offs_d.index_select(0, idx).contiguous(),
                           lens_d.index_select(0, idx).contiguous(), max_len, hq, hkv, d, 1.0 / math.sqrt(d))
        ob = bits(o)
        return [ob[j:j + 1] for j in range(len(reqs))]

    calls = harness.plan(range(64), [1, 2, 4, 7, 8, 16, 32, 33, 64], repeats=10, batch_repeats=2, seed=405)
    rep = harness.run(backend, calls, log=lambda m: None if m.startswith("alone") else announce("decode", m))
    print("decode requests:", rep.summary())
    assert rep.invariant and rep.identical_pct == 100.0, rep.summary()
    assert len(rep.distinct) == 64 and min(rep.observations.values()) >= 10
