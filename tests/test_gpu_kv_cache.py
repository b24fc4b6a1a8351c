"""GPU tests of the quantised, paged KV cache (through the C-ABI).

bi_kv_append_q8 must store exactly the oracle's int8 codes and float32 scales.
Attention over the paged int8 cache must give bit for bit what the bf16
kernels give on the dequantised values laid out contiguously (prefill whole
and chunked, decode in prefill order), must not depend on where the pages are,
and decode must equal prefill for the same query.  Parity against the oracle's
attention on the dequantised values to the usual tolerance.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import kv_cache as KV
from invariant_deterministic_amd import bi, synth
from tests.gpu_util import announce, assert_bitwise, bits, dev, device
from tests.util import assert_within_tolerance

pytestmark = pytest.mark.gpu
PAGE = 64


def kv_rows(rng, n, hkv, d):
    """bf16 rows with per-(row, head) magnitudes spread over 2^+-8, some zero and constant heads."""
    x = rng.standard_normal((n, hkv, d)) * np.exp2(rng.uniform(-8, 8, (n, hkv, 1)))
    x[::17, 0] = 0.0
    x[5::23, -1] = -0.375
    return oracle.bf16_round(x)


@pytest.mark.parametrize("hkv,d", [(8, 128), (4, 64)])
def test_kv_append_matches_oracle(hkv, d):
    device()
    rng = np.random.default_rng(9000 + d)
    n = 700
    k, v = kv_rows(rng, n, hkv, d), kv_rows(rng, n, hkv, d)
    pool = bi.KvPoolQ8(16, hkv, d)
    dst = rng.permutation(16 * PAGE)[:n].astype(np.int64)
    announce("kv append q8", hkv, d)
    bi.kv_append_q8(pool, dev(k), dev(v), torch.from_numpy(dst).cuda())
    torch.cuda.synchronize()
    for name, x, codes, scales in (("k", k, pool.k, pool.ks), ("v", v, pool.v, pool.vs)):
        q, s = KV.quantize(x)
        assert np.array_equal(codes.cpu().numpy()[dst], q), f"{name} codes"
        assert np.array_equal(scales.cpu().numpy()[dst].view(np.uint32), s.view(np.uint32)), f"{name} scales"


def build_sequence(rng, L, hkv, d, pages_in_pool):
    """A sequence's K/V quantised into random distinct pages; returns the pool, its table and
    the oracle's dequantised K/V in logical order."""
    k, v = kv_rows(rng, L, hkv, d), kv_rows(rng, L, hkv, d)
    npg = -(-L // PAGE)
    table = rng.permutation(pages_in_pool)[:npg].astype(np.int32)
    pool = bi.KvPoolQ8(pages_in_pool, hkv, d)
    rows = table[np.arange(L) // PAGE].astype(np.int64) * PAGE + np.arange(L) % PAGE
    bi.kv_append_q8(pool, dev(k), dev(v), torch.from_numpy(rows).cuda())
    kd = KV.dequantize(*KV.quantize(k))
    vd = KV.dequantize(*KV.quantize(v))
    return pool, table, kd, vd, (k, v)


@pytest.mark.parametrize("hq,hkv,d", [(32, 8, 128), (4, 4, 64)])
def test_prefill_paged_q8(hq, hkv, d):
    device()
    rng = np.random.default_rng(9100 + d)
    L = 700
    pool, table, kd, vd, raw = build_sequence(rng, L, hkv, d, 40)
    q = synth.normal_bf16(9101 + d, (L, hq * d))
    scale = 1.0 / math.sqrt(d)
    tbl = torch.from_numpy(table).cuda()
    announce("prefill paged q8", hq, hkv, d)
    got = bits(bi.attn_prefill_paged_q8(dev(q), pool, tbl, 0, hq, scale))
    ref = bits(bi.attn_prefill(dev(q), dev(kd), dev(vd), 0, hq, hkv, d, scale))
    assert_bitwise(got, ref, "paged q8 prefill vs bf16 prefill on the dequantised cache")
    chunk = bits(bi.attn_prefill_paged_q8(dev(q[300:]), pool, tbl, 300, hq, scale))
    assert_bitwise(chunk, got[300:], "chunked")
    # the same sequence in other pages
    pool2, table2, _, _, _ = build_sequence(np.random.default_rng(9100 + d), L, hkv, d, 57)
    assert not np.array_equal(table2[:len(table)], table)
    got2 = bits(bi.attn_prefill_paged_q8(dev(q), pool2, torch.from_numpy(table2).cuda(), 0, hq, scale))
    assert_bitwise(got2, got, "other page placement")
    # parity with the oracle on the dequantised values (sampled rows)
    rows = np.array([0, 63, 64, 299, 699])
    att = oracle.attention(q.reshape(L, hq, d)[rows], kd, vd, rows, np.float32(scale))
    assert_within_tolerance(got[rows], att.reshape(len(rows), -1), "paged q8 prefill parity")


def test_decode_paged_q8():
    device()
    hq, hkv, d = 32, 8, 128
    rng = np.random.default_rng(9200)
    lens = np.array([1, 63, 64, 65, 500, 1000, 2049])
    B = len(lens)
    max_pages = -(-int(lens.max()) // PAGE)
    pool = bi.KvPoolQ8(200, hkv, d)
    perm = rng.permutation(200)
    tables = np.zeros((B, max_pages), np.int32)
    kds, vds, qs = [], [], []
    used = 0
    for b, L in enumerate(lens):
        npg = -(-int(L) // PAGE)
        tables[b, :npg] = perm[used:used + npg]
        used += npg
        k, v = kv_rows(rng, L, hkv, d), kv_rows(rng, L, hkv, d)
        rows = tables[b, np.arange(L) // PAGE].astype(np.int64) * PAGE + np.arange(L) % PAGE
        bi.kv_append_q8(pool, dev(k), dev(v), torch.from_numpy(rows).cuda())
        kds.append(KV.dequantize(*KV.quantize(k)))
        vds.append(KV.dequantize(*KV.quantize(v)))
        qs.append(synth.normal_bf16(9201 + b, (int(L), hq * d)))
    scale = 1.0 / math.sqrt(d)
    tbl = torch.from_numpy(tables).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    q_last = np.stack([qs[b][-1] for b in range(B)])
    announce("decode paged q8", list(lens))
    dec = bits(bi.attn_decode_paged_q8(dev(q_last), pool, tbl, ld, int(lens.max()), hq, scale))
    # bf16 decode in prefill order over the dequantised values, packed contiguously
    kc = np.concatenate(kds)
    vc = np.concatenate(vds)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    ref = bits(bi.attn_decode_prefill_order(dev(q_last), dev(kc), dev(vc), torch.from_numpy(offs).cuda(), ld,
                                            int(lens.max()), hq, hkv, d, scale))
    assert_bitwise(dec, ref, "paged q8 decode vs bf16 decode on the dequantised cache")
    for b, L in enumerate(lens):
        pf = bits(bi.attn_prefill_paged_q8(dev(qs[b]), pool, torch.from_numpy(tables[b]).cuda(), 0, hq, scale))
        assert_bitwise(dec[b], pf[L - 1], f"L={L}: paged decode vs paged prefill")
        att = oracle.decode_attention(q_last[b].reshape(hq, d), kds[b], vds[b], np.float32(scale))
        assert_within_tolerance(dec[b], att.reshape(-1), f"L={L}: parity")
    # alone vs batched with a launch order
    order = torch.from_numpy(np.argsort(-lens, kind="stable").astype(np.int32)).cuda()
    again = bits(bi.attn_decode_paged_q8(dev(q_last), pool, tbl, ld, int(lens.max()), hq, scale, order=order))
    assert_bitwise(again, dec, "with an order")
    for b in (0, 4, 6):
        one = bits(bi.attn_decode_paged_q8(dev(q_last[b:b + 1]), pool, tbl[b:b + 1], ld[b:b + 1], int(lens[b]), hq,
                                           scale))
        assert_bitwise(one[0], dec[b], f"request {b} alone")


def test_decode_paged_q8_bench_workload():
    """The int8 paged decode at the size and launch bench.py times: 256 requests with KV
    lengths 513..8193, 32/8 heads x 128, 64-token pages in random order, requests longest
    first.  Every request is bitwise equal to the bf16 prefill-order decode over the same cache
    de-quantised (bf16(float(code) * scale)) and laid out contiguously, and to the same launch
    without the order; sampled requests equal their run alone, their codes and scales equal the
    oracle's quantisation of the same seeded rows, and their outputs are within tolerance of the
    oracle's attention."""
    device()
    hq, hkv, d, B = 32, 8, 128, 256
    lens = synth.uniform_ints(501, B, 512, 8192) + 1
    npg = (lens + PAGE - 1) // PAGE
    total = int(npg.sum())
    perm = np.random.default_rng(1400).permutation(total).astype(np.int32)
    tables = np.zeros((B, int(npg.max())), np.int32)
    used, rows = 0, []
    for b in range(B):
        tables[b, :npg[b]] = perm[used:used + npg[b]]
        used += int(npg[b])
        rows.append(tables[b, np.arange(lens[b]) // PAGE].astype(np.int64) * PAGE + np.arange(lens[b]) % PAGE)
    rows_np = np.concatenate(rows)
    rows_d = torch.from_numpy(rows_np).cuda()
    n = rows_np.size
    CH = 1 << 18   # the seeded rows come in chunks of CH, each drawn on the device
    pool = bi.KvPoolQ8(total, hkv, d)
    for s0 in range(0, n, CH):
        m = min(n - s0, CH)
        bi.kv_append_q8(pool, synth.normal_bf16_device(1401 + s0, (m, hkv, d)),
                        synth.normal_bf16_device(1402 + s0, (m, hkv, d)), rows_d[s0:s0 + m].contiguous())
    q_host = synth.normal_bf16(402, (B, hq * d))
    q = dev(q_host)
    tbl = torch.from_numpy(tables).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    order = torch.from_numpy(np.argsort(-lens, kind="stable").astype(np.int32)).cuda()
    mx, scale = int(lens.max()), 1.0 / math.sqrt(d)
    announce("decode paged q8, bench workload: 256 requests, KV 513..8193")
    dec = bits(bi.attn_decode_paged_q8(q, pool, tbl, ld, mx, hq, scale, order=order))
    assert_bitwise(bits(bi.attn_decode_paged_q8(q, pool, tbl, ld, mx, hq, scale)), dec, "without the launch order")
    # the de-quantised cache, contiguous in request order, through the bf16 prefill-order decode
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)

    def dequant(codes, sc):
        return (codes[rows_d].float() * sc[rows_d].unsqueeze(-1)).to(torch.bfloat16)

    kdq, vdq = dequant(pool.k, pool.ks), dequant(pool.v, pool.vs)
    ref = bits(bi.attn_decode_prefill_order(q, kdq, vdq, torch.from_numpy(offs).cuda(), ld, mx, hq, hkv, d, scale,
                                            order=order))
    assert_bitwise(dec, ref, "paged q8 vs bf16 prefill-order decode on the de-quantised cache")
    del kdq, vdq, ref

    def seeded_rows(seed0, lo, hi):
        """Rows lo..hi-1 of the seeded stream (chunks of CH rows drawn with seed seed0 + chunk start)."""
        parts = []
        for s0 in range(lo // CH * CH, hi, CH):
            m = min(n - s0, CH)
            parts.append(bits(synth.normal_bf16_device(seed0 + s0, (m, hkv, d))[max(lo, s0) - s0:min(hi, s0 + m) - s0]))
        return np.concatenate(parts)

    for b in (int(np.argmax(lens)), int(np.argmin(lens)), 17, 200):
        announce("decode paged q8, bench workload, request", b, "L =", int(lens[b]))
        one = bits(bi.attn_decode_paged_q8(q[b:b + 1], pool, tbl[b:b + 1], ld[b:b + 1], int(lens[b]), hq, scale))
        assert_bitwise(one[0], dec[b], f"request {b} alone")
        lo, hi = int(offs[b]), int(offs[b] + lens[b])
        rb = torch.from_numpy(rows_np[lo:hi]).cuda()
        kq, ks = KV.quantize(seeded_rows(1401, lo, hi))
        vq, vs = KV.quantize(seeded_rows(1402, lo, hi))
        assert np.array_equal(kq, pool.k[rb].cpu().numpy()) and np.array_equal(vq, pool.v[rb].cpu().numpy())
        assert np.array_equal(ks.view(np.uint32), pool.ks[rb].cpu().numpy().view(np.uint32))
        assert np.array_equal(vs.view(np.uint32), pool.vs[rb].cpu().numpy().view(np.uint32))
        att = oracle.decode_attention(q_host[b].reshape(hq, d), KV.dequantize(kq, ks), KV.dequantize(vq, vs),
                                      np.float32(scale))
        assert_within_tolerance(dec[b], att.reshape(-1), f"request {b} parity")
