"""GPU tests of bi_attn_decode_prefill_order and of the block's prefill-order decode mode.

A token's bits must not depend on whether it was prefilled, verified inside a
drafted chunk or decoded alone ("Receipts", opening paragraph: independent of
run-ahead drafting; M-0002 "Limitations": speculative decoding is open work).
Checked bitwise: decode in prefill order == the prefill kernel's row for the
same query (whole sequence in one pass, a one-token chunk, a drafted chunk),
at lengths around every block and half-block boundary; alone == batched ==
reordered; and through bi_block_forward, a decoded or draft-verified token's
output row == its row when the whole sequence is prefilled.  Parity against
the oracle to the usual tolerance.
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

LENS = np.array([1, 2, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 300, 1000, 2049])


def packed_kv(lens, hkv, d, seed, spread=0.0):
    """Packed K/V ~ N(0,1); with spread > 0 every (key, head) row of K is scaled by
    2^U(-spread, spread), so block maxima jump and the online softmax rescales often."""
    total = int(np.sum(lens))
    k = synth.normal_bf16_device(seed, (total, hkv, d))
    if spread:
        rng = np.random.default_rng(seed + 7)
        mag = torch.from_numpy(np.exp2(rng.uniform(-spread, spread, (total, hkv, 1))).astype(np.float32)).cuda()
        k = (k.float() * mag).to(torch.bfloat16)
    v = synth.normal_bf16_device(seed + 1, (total, hkv, d))
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return k, v, offs


def decode_po(q, k, v, offs, lens, max_len, hq, hkv, d, order=None):
    return bi.attn_decode_prefill_order(
        q, k, v, torch.from_numpy(np.asarray(offs, np.int64)).cuda(),
        torch.from_numpy(np.asarray(lens, np.int32)).cuda(), max_len, hq, hkv, d, 1.0 / math.sqrt(d),
        order=None if order is None else torch.from_numpy(np.asarray(order, np.int32)).cuda())


@pytest.mark.parametrize("hq,hkv,d,spread", [(32, 8, 128, 0.0), (4, 4, 64, 0.0), (8, 4, 128, 0.0), (16, 4, 64, 0.0),
                                            (32, 8, 128, 8.0), (4, 4, 64, 3.0), (16, 4, 64, 6.0)])
def test_decode_equals_prefill_bitwise(hq, hkv, d, spread):
    device()
    lens = LENS
    announce("decode in prefill order vs prefill", hq, hkv, d, spread)
    k, v, offs = packed_kv(lens, hkv, d, 7000 + d + hq, spread)
    scale = 1.0 / math.sqrt(d)
    qs = [dev(synth.normal_bf16(7002 + 17 * b + hq, (int(L), hq * d))) for b, L in enumerate(lens)]
    q_last = torch.stack([qs[b][-1] for b in range(len(lens))])
    dec = bits(decode_po(q_last, k, v, offs, lens, int(lens.max()), hq, hkv, d))
    for b, L in enumerate(lens):
        L = int(L)
        kc, vc = k[offs[b]:offs[b] + L], v[offs[b]:offs[b] + L]
        whole = bits(bi.attn_prefill(qs[b], kc, vc, 0, hq, hkv, d, scale))
        assert_bitwise(dec[b], whole[L - 1], f"L={L}: decode vs whole-sequence prefill")
        one = bits(bi.attn_prefill(qs[b][L - 1:], kc, vc, L - 1, hq, hkv, d, scale))
        assert_bitwise(dec[b], one[0], f"L={L}: decode vs one-token prefill chunk")
        s = max(0, L - 4)
        draft = bits(bi.attn_prefill(qs[b][s:], kc, vc, s, hq, hkv, d, scale))
        assert_bitwise(dec[b], draft[-1], f"L={L}: decode vs drafted chunk")


@pytest.mark.parametrize("spread", [0.0, 4.0])
def test_decode_prefill_order_parity(spread):
    device()
    hq, hkv, d = 32, 8, 128
    lens = np.array([1, 33, 64, 97, 255, 1000, 4097])
    announce("decode in prefill order parity", list(lens), spread)
    k, v, offs = packed_kv(lens, hkv, d, 7100, spread)
    q = synth.normal_bf16(7102, (len(lens), hq * d))
    o = bits(decode_po(dev(q), k, v, offs, lens, int(lens.max()), hq, hkv, d))
    kb, vb = bits(k), bits(v)
    for b, L in enumerate(lens):
        ref = oracle.decode_attention(q[b].reshape(hq, d), kb[offs[b]:offs[b] + L], vb[offs[b]:offs[b] + L],
                                      np.float32(1.0 / math.sqrt(d)))
        assert_within_tolerance(o[b], ref.reshape(-1), f"decode in prefill order b={b} L={L}")
        if L == 1:
            assert_bitwise(o[b].reshape(hq, d), np.repeat(vb[offs[b]], hq // hkv, axis=0), "L=1 gives v")


def test_decode_prefill_order_batch_invariance_and_order():
    device()
    hq, hkv, d = 32, 8, 128
    lens = synth.uniform_ints(7200, 24, 1, 3000)
    k, v, offs = packed_kv(lens, hkv, d, 7201)
    q = dev(synth.normal_bf16(7203, (24, hq * d)))
    alone = [bits(decode_po(q[b:b + 1], k, v, offs[b:b + 1], lens[b:b + 1], 3000, hq, hkv, d))[0] for b in range(24)]
    rng = np.random.default_rng(7204)
    for B in (3, 16, 24):
        for rep in range(2):
            idx = rng.choice(24, size=B, replace=False)
            order = rng.permutation(B) if rep else np.argsort(-lens[idx], kind="stable")
            announce("decode in prefill order, batch", B, rep)
            o = bits(decode_po(q[torch.from_numpy(idx).cuda()], k, v, offs[idx], lens[idx], 3000 + 100 * rep,
                               hq, hkv, d, order=order))
            for j, b in enumerate(idx):
                assert_bitwise(o[j], alone[b], f"request {b} in batch {B}")


def test_decode_prefill_order_length_outside_grid_is_nan():
    device()
    hq, hkv, d = 8, 4, 64
    lens = np.array([40, 100, 70])
    k, v, offs = packed_kv(lens, hkv, d, 7300)
    q = dev(synth.normal_bf16(7302, (3, hq * d)))
    ok = bits(decode_po(q, k, v, offs, lens, 100, hq, hkv, d))
    announce("decode in prefill order, length beyond max_kv_len")
    o = bits(decode_po(q, k, v, offs, lens, 80, hq, hkv, d))   # request 1 (L = 100) is outside the grid
    assert np.all(o[1] == 0x7FC0)
    assert_bitwise(o[[0, 2]], ok[[0, 2]], "other requests unaffected")


# --------------------------------------------------------------- block level
CFG_DENSE = dict(hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728, eps=1e-6, rope_theta=1e6)
CFG_TINY = dict(hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=0, eps=1e-6, rope_theta=0.0)


def make_block(cfg, base, prefill_order=True):
    H, hq, hkv, d, F = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn"))
    w = dict(gamma1=synth.ones_bf16(H), gamma2=synth.ones_bf16(H),
             w_qkv=synth.normal_bf16(base + 2, ((hq + 2 * hkv) * d, H), 0.02),
             w_o=synth.normal_bf16(base + 3, (H, hq * d), 0.02))
    if F:
        w["w_gate_up"] = synth.normal_bf16(base + 4, (2 * F, H), 0.02)
        w["w_down"] = synth.normal_bf16(base + 6, (H, F), 0.02)
    bc = bi.BlockConfig(H, hq, hkv, d, F, cfg["eps"], cfg["rope_theta"], decode_prefill_order=prefill_order)
    return bi.Block(bc, {key: dev(val) for key, val in w.items()})


@pytest.mark.parametrize("cfg", [CFG_DENSE, CFG_TINY], ids=["dense", "tiny"])
def test_block_decoded_token_equals_prefilled(cfg):
    """Sequence A: n + 6 tokens prefilled in one pass.  Then the same tokens as a
    prefill of n, two decode steps, a drafted chunk of 3 and one more decode, run
    next to other requests (decodes at other lengths and a prefill chunk); every
    row must equal A's."""
    device()
    H, hkv, d = cfg["hidden"], cfg["n_kv_heads"], cfg["head_dim"]
    blk = make_block(cfg, 7400)
    n = 189
    total = n + 6
    x = synth.normal_bf16(7401, (total, H))
    cap = 8192
    kp = torch.zeros((cap, hkv, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    announce("block prefill order: whole pass", total)
    y_all = bits(blk.forward(dev(x), [dict(q_len=total, ctx_len=0, kv_base=0)], kp, vp)[0])
    # other requests: cached keys at fixed pool regions, written by a prefill of their own
    other_lens = [37, 700, 64]
    other_x = [synth.normal_bf16(7410 + i, (L + 1, H)) for i, L in enumerate(other_lens)]
    for i, L in enumerate(other_lens):
        blk.forward(dev(other_x[i][:L]), [dict(q_len=L, ctx_len=0, kv_base=2048 * (i + 1))], kp, vp)
    pf_x = synth.normal_bf16(7420, (50, H))
    base = 1024
    announce("block prefill order: prefix", n)
    y = bits(blk.forward(dev(x[:n]), [dict(q_len=n, ctx_len=0, kv_base=base)], kp, vp)[0])
    assert_bitwise(y, y_all[:n], "prefix rows")
    pos = n
    for step, q_len in enumerate((1, 1, 3, 1)):
        seqs = [dict(q_len=1, ctx_len=L, kv_base=2048 * (i + 1)) for i, L in enumerate(other_lens)]
        seqs.insert(1, dict(q_len=q_len, ctx_len=pos, kv_base=base))
        seqs.append(dict(q_len=50, ctx_len=0, kv_base=7000 + 64 * step))
        rows = [other_x[0][other_lens[0]:other_lens[0] + 1], x[pos:pos + q_len],
                other_x[1][other_lens[1]:other_lens[1] + 1], other_x[2][other_lens[2]:other_lens[2] + 1], pf_x]
        announce("block prefill order: step", step, "q_len", q_len)
        yb = bits(blk.forward(dev(np.concatenate(rows)), seqs, kp, vp)[0])
        assert_bitwise(yb[1:1 + q_len], y_all[pos:pos + q_len], f"step {step}: tokens {pos}..{pos + q_len - 1}")
        pos += q_len
    assert pos == total
