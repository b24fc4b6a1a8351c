"""GPU parity and invariance of bi_attn_decode, bi_attn_prefill, bi_rope_kv,
bi_add and bi_swiglu (through the C-ABI).

Decode: fixed 256-key units merged in runs of 8 (2048 keys), then across runs;
every request's bits identical alone and in any batch, at unit and run
boundaries and for L = 1 (o = v exactly); requests outside 1 .. max_kv_len
give NaN without disturbing the others.  Prefill: chunking
invariance (one pass vs chunks, chunks starting mid-tile), t = 0 gives v0.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import bi, synth
from tests.gpu_util import announce, assert_bitwise, bits, dev, device
from tests.util import assert_within_tolerance

pytestmark = pytest.mark.gpu


def packed_kv(lens, hkv, d, seed):
    total = int(np.sum(lens))
    k = synth.normal_bf16_device(seed, (total, hkv, d))
    v = synth.normal_bf16_device(seed + 1, (total, hkv, d))
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return k, v, offs


def run_decode(q, k, v, offs, lens, max_len, hq, hkv, d):
    return bi.attn_decode(q, k, v, torch.from_numpy(np.asarray(offs, np.int64)).cuda(),
                          torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max_len, hq, hkv, d,
                          1.0 / math.sqrt(d))


# ------------------------------------------------------------------- decode
@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (4, 4, 64), (16, 2, 128), (8, 4, 64)])
def test_decode_parity_split_boundaries(hq, hkv, d):
    device()
    lens = np.array([1, 2, 255, 256, 257, 511, 512, 513, 1000, 2048, 2049, 2304, 4097])
    announce("decode parity", hq, hkv, d, list(lens))
    k, v, offs = packed_kv(lens, hkv, d, 4000 + d + hq)
    q = synth.normal_bf16(4002 + hq, (len(lens), hq * d))
    o = bits(run_decode(dev(q), k, v, offs, lens, int(lens.max()), hq, hkv, d))
    kb, vb = bits(k), bits(v)
    for b, L in enumerate(lens):
        ref = oracle.decode_attention(q[b].reshape(hq, d), kb[offs[b]:offs[b] + L], vb[offs[b]:offs[b] + L],
                                      np.float32(1.0 / math.sqrt(d)))
        assert_within_tolerance(o[b], ref.reshape(-1), f"decode b={b} L={L}")
        if L == 1:
            g = hq // hkv
            assert_bitwise(o[b].reshape(hq, d), np.repeat(vb[offs[b]], g, axis=0), "decode L=1 gives v")


def test_decode_batch_invariance():
    device()
    hq, hkv, d = 32, 8, 128
    lens = synth.uniform_ints(4100, 24, 1, 4096)
    k, v, offs = packed_kv(lens, hkv, d, 4101)
    q = dev(synth.normal_bf16(4103, (24, hq * d)))
    max_len = 4096
    alone = [bits(run_decode(q[b:b + 1], k, v, offs[b:b + 1], lens[b:b + 1], max_len, hq, hkv, d))[0]
             for b in range(24)]
    rng = np.random.default_rng(4104)
    for B in (2, 5, 16, 24):
        for rep in range(3):
            idx = rng.choice(24, size=B, replace=False)
            announce("decode invariance", B, rep)
            # a larger max_kv_len (grid) must not matter either
            o = bits(run_decode(q[torch.from_numpy(idx).cuda()], k, v, offs[idx], lens[idx],
                                max_len + 256 * rep, hq, hkv, d))
            for j, b in enumerate(idx):
                assert_bitwise(o[j], alone[b], f"decode request {b} in batch {B}")


def test_decode_many_requests_and_bad_lengths():
    """1500 requests (the standalone entry point lists their runs on the device, 1024 requests
    at a time): lengths 0 and above max_kv_len give NaN rows, every other row equals the
    request decoded alone."""
    device()
    hq, hkv, d = 4, 1, 64
    B, max_len = 1500, 2600
    lens = synth.uniform_ints(4300, B, 1, max_len)
    bad = np.array([3, 700, 1024, 1499])
    lens[bad[:2]] = 0
    lens[bad[2:]] = max_len + 1
    kv_lens = np.maximum(lens, 1)
    k, v, offs = packed_kv(kv_lens, hkv, d, 4301)
    q = dev(synth.normal_bf16(4303, (B, hq * d)))
    announce("decode B=1500 with bad lengths")
    o = run_decode(q, k, v, offs, lens, max_len, hq, hkv, d).float().cpu().numpy()
    ob = bits(run_decode(q, k, v, offs, lens, max_len, hq, hkv, d))
    assert np.isnan(o[bad]).all()
    good = np.setdiff1d(np.arange(B), bad)
    assert np.isfinite(o[good]).all()
    for b in np.random.default_rng(4304).choice(good, 12, replace=False):
        alone = bits(run_decode(q[b:b + 1], k, v, offs[b:b + 1], lens[b:b + 1], max_len, hq, hkv, d))[0]
        assert_bitwise(ob[b], alone, f"request {b} (L={lens[b]}) alone vs B=1500")


def test_decode_config4_full_batch():
    """B = 64, L ~ U{1..32768}: every request vs the oracle; sampled requests alone vs batched
    (all 64, in batches of many sizes and orders, run through the invariance harness in
    test_gpu_invariance.py)."""
    device()
    hq, hkv, d = 32, 8, 128
    lens = synth.uniform_ints(401, 64, 1, 32768)
    k, v, offs = packed_kv(lens, hkv, d, 403)
    q = synth.normal_bf16(402, (64, hq * d))
    qd = dev(q)
    announce("decode config4 B=64")
    o = bits(run_decode(qd, k, v, offs, lens, 32768, hq, hkv, d))
    for rep in range(3):
        assert_bitwise(bits(run_decode(qd, k, v, offs, lens, 32768, hq, hkv, d)), o, "decode repeat")
    samp = set(int(b) for b in np.random.default_rng(404).choice(64, 6, replace=False))
    announce("decode config4: all 64 requests vs the oracle")
    for b in range(64):
        sl = slice(int(offs[b]), int(offs[b] + lens[b]))
        kb = bits(k[sl]); vb = bits(v[sl])
        ref = oracle.decode_attention(q[b].reshape(hq, d), kb, vb, np.float32(1 / math.sqrt(d)))
        assert_within_tolerance(o[b], ref.reshape(-1), f"decode config4 b={b} (L={lens[b]})")
        if b in samp:
            alone = bits(run_decode(qd[b:b + 1], k, v, offs[b:b + 1], lens[b:b + 1], int(lens[b]), hq, hkv, d))[0]
            assert_bitwise(alone, o[b], f"decode config4 request {b} alone vs B=64")


def test_decode_length_32768_boundary():
    device()
    hq, hkv, d = 32, 8, 128
    lens = np.array([32768, 32767, 32513])
    k, v, offs = packed_kv(lens, hkv, d, 4200)
    q = synth.normal_bf16(4202, (3, hq * d))
    announce("decode L=32768")
    o = bits(run_decode(dev(q), k, v, offs, lens, 32768, hq, hkv, d))
    for b in range(3):
        sl = slice(int(offs[b]), int(offs[b] + lens[b]))
        ref = oracle.decode_attention(q[b].reshape(hq, d), bits(k[sl]), bits(v[sl]), np.float32(1 / math.sqrt(d)))
        assert_within_tolerance(o[b], ref.reshape(-1), f"decode L={lens[b]}")


# ------------------------------------------------------------------ prefill
def prefill_case(T_total, hq, hkv, d, seed):
    q = synth.normal_bf16(seed, (T_total, hq * d))
    k = synth.normal_bf16(seed + 1, (T_total, hkv, d))
    v = synth.normal_bf16(seed + 2, (T_total, hkv, d))
    return q, k, v


@pytest.mark.parametrize("T,q_start,hq,hkv,d", [(300, 0, 32, 8, 128), (250, 250, 32, 8, 128),
                                                (128, 0, 4, 4, 64), (200, 77, 8, 4, 64), (129, 0, 16, 8, 128)])
def test_prefill_parity(T, q_start, hq, hkv, d):
    device()
    announce("prefill parity", T, q_start, hq, hkv, d)
    q, k, v = prefill_case(q_start + T, hq, hkv, d, 5000 + T + q_start)
    sc = np.float32(1 / math.sqrt(d))
    o = bits(bi.attn_prefill(dev(q[q_start:]), dev(k), dev(v), q_start, hq, hkv, d, float(sc)))
    ref = oracle.attention(q[q_start:].reshape(T, hq, d), k, v, np.arange(q_start, q_start + T), sc)
    assert_within_tolerance(o, ref.reshape(T, -1), f"prefill T={T} start={q_start}")
    if q_start == 0:
        g = hq // hkv
        assert_bitwise(o[0].reshape(hq, d), np.repeat(v[0], g, axis=0), "prefill t=0 gives v0")



def test_prefill_long_context():
    """A short chunk at the end of a 30000-token context: parity on every row, and the same
    bits when the chunk itself is split (the key blocks are aligned to position 0)."""
    device()
    hq, hkv, d = 32, 8, 128
    q_start, T = 30000, 100
    q = synth.normal_bf16(5300, (T, hq * d))
    kd = synth.normal_bf16_device(5301, (q_start + T, hkv, d))
    vd = synth.normal_bf16_device(5302, (q_start + T, hkv, d))
    sc = np.float32(1 / math.sqrt(d))
    announce("prefill long context", q_start, T)
    qd = dev(q)
    o = bits(bi.attn_prefill(qd, kd, vd, q_start, hq, hkv, d, float(sc)))
    parts = [bits(bi.attn_prefill(qd[:37], kd, vd, q_start, hq, hkv, d, float(sc))),
             bits(bi.attn_prefill(qd[37:], kd, vd, q_start + 37, hq, hkv, d, float(sc)))]
    assert_bitwise(np.concatenate(parts), o, "prefill long context split 37 + 63")
    ref = oracle.attention(q.reshape(T, hq, d), bits(kd), bits(vd), np.arange(q_start, q_start + T), sc)
    assert_within_tolerance(o, ref.reshape(T, -1), f"prefill T={T} start={q_start}")

@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (4, 4, 64)])
def test_prefill_chunk_invariance(hq, hkv, d):
    device()
    T = 1000
    q, k, v = prefill_case(T, hq, hkv, d, 5100 + d)
    qd, kd, vd = dev(q), dev(k), dev(v)
    sc = 1 / math.sqrt(d)
    whole = bits(bi.attn_prefill(qd, kd, vd, 0, hq, hkv, d, sc))
    for chunks in ([250] * 4, [100, 157, 743], [64, 64, 872], [1, 999], [999, 1], [500, 500]):
        announce("prefill chunking", chunks)
        parts, s0 = [], 0
        for c in chunks:
            # the cache holds only the keys written so far (rest poisoned with NaN)
            kc = kd.clone(); vc = vd.clone()
            kc[s0 + c:] = float("nan"); vc[s0 + c:] = float("nan")
            parts.append(bits(bi.attn_prefill(qd[s0:s0 + c], kc, vc, s0, hq, hkv, d, sc)))
            s0 += c
        assert_bitwise(np.concatenate(parts), whole, f"prefill chunks {chunks}")
    ref = oracle.attention(q.reshape(T, hq, d), k, v, np.arange(T), np.float32(sc))
    assert_within_tolerance(whole, ref.reshape(T, -1), "prefill T=1000 parity")


def test_prefill_4000_chunkings():
    device()
    hq, hkv, d = 32, 8, 128
    T = 4000
    q = synth.normal_bf16_device(5200, (T, hq * d))
    k = synth.normal_bf16_device(5201, (T, hkv, d))
    v = synth.normal_bf16_device(5202, (T, hkv, d))
    sc = 1 / math.sqrt(d)
    announce("prefill 4000 whole")
    whole = bits(bi.attn_prefill(q, k, v, 0, hq, hkv, d, sc))
    for c in (250, 1000):
        announce("prefill 4000 chunk", c)
        parts = [bits(bi.attn_prefill(q[s:s + c], k, v, s, hq, hkv, d, sc)) for s in range(0, T, c)]
        assert_bitwise(np.concatenate(parts), whole, f"prefill 4000 in chunks of {c}")
    rows = np.array([0, 1, 63, 64, 255, 256, 1999, 3999])
    kb, vb, qb = bits(k), bits(v), bits(q)
    ref = oracle.attention(qb[rows].reshape(len(rows), hq, d), kb, vb, rows, np.float32(sc))
    assert_within_tolerance(whole[rows], ref.reshape(len(rows), -1), "prefill 4000 sampled rows")


# ----------------------------------------------------------- elementwise
def test_add_bitwise():
    device()
    announce("add")
    x = synth.normal_bf16(6000, (513, 2560))
    o = synth.normal_bf16(6001, (513, 2560), 0.3)
    assert_bitwise(bits(bi.add(dev(x), dev(o))), oracle.residual_add(x, o), "residual add")


def test_swiglu_parity():
    device()
    announce("swiglu")
    gu = synth.normal_bf16(6100, (300, 2 * 9728), 2.0)
    act = bits(bi.swiglu(dev(gu)))
    assert_within_tolerance(act, oracle.swiglu(gu[:, :9728], gu[:, 9728:]), "swiglu")


@pytest.mark.parametrize("hq,hkv,d,theta", [(32, 8, 128, 1e6), (4, 4, 64, 1e4), (4, 4, 64, 0.0)])
def test_rope_kv(hq, hkv, d, theta):
    device()
    announce("rope_kv", hq, hkv, d, theta)
    rows = 300
    qkv = synth.normal_bf16(6200 + d, (rows, (hq + 2 * hkv) * d))
    pos = np.concatenate([np.arange(0, 100), np.arange(7990, 8190), ]).astype(np.int32)
    kv_row = (np.arange(rows) * 3 + 5).astype(np.int64)  # scattered rows in the pool
    pool_rows = int(kv_row.max()) + 1
    kp = torch.zeros((pool_rows, hkv, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    qo = bi.rope_kv(dev(qkv), torch.from_numpy(pos).cuda(), torch.from_numpy(kv_row).cuda(), kp, vp,
                    hq, hkv, d, theta)
    qo, kpb, vpb = bits(qo), bits(kp), bits(vp)
    x = qkv.reshape(rows, hq + 2 * hkv, d)
    if theta:
        q_ref = oracle.rope(x[:, :hq], pos, theta).reshape(rows, -1)
        k_ref = oracle.rope(x[:, hq:hq + hkv], pos, theta)
        assert_within_tolerance(qo, q_ref, "rope q")
        assert_within_tolerance(kpb[kv_row], k_ref, "rope k")
        p0 = pos == 0
        assert_bitwise(qo[p0], x[p0, :hq].reshape(int(p0.sum()), -1), "rope at position 0 is identity")
    else:
        assert_bitwise(qo, x[:, :hq].reshape(rows, -1), "no-rope q copy")
        assert_bitwise(kpb[kv_row], x[:, hq:hq + hkv], "no-rope k copy")
    assert_bitwise(vpb[kv_row], x[:, hq + hkv:], "v append")
    untouched = np.setdiff1d(np.arange(pool_rows), kv_row)
    assert np.all(kpb[untouched] == 0) and np.all(vpb[untouched] == 0)
