"""GPU tests of bi_block_forward: parity against the oracle (end-to-end and
stage by stage) and bitwise invariance of every request's rows across batch
size, batch position, prefill chunking and repeats, counted by the invariance
harness (distinct outputs per request over alone, batched, permuted and
repeated runs).  Every workspace and output is filled with NaN bytes before
each forward, so a stage read before it is written shows up.

Shapes: the tiny block (hidden 256, 4 heads of 64, no RoPE, no FFN), the dense
Qwen3-4B-shaped block (hidden 2560, 32/8 heads of 128, RoPE 1e6, SwiGLU 9728)
and the int4 block (hidden 4096, FFN 12288) on a mixed step of up to 256
decodes plus a 2048-token prefill chunk.
"""
import hashlib
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import kv_cache as KV
from invariant_deterministic_amd import bi, harness, synth
from tests.gpu_util import announce, assert_bitwise, bits, dev, device, forward_poisoned, split_rows
from tests.util import assert_rowwise_norm, assert_within_tolerance

pytestmark = pytest.mark.gpu

CFG1 = dict(hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=0, eps=1e-6, rope_theta=0.0)
CFG3 = dict(hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728, eps=1e-6, rope_theta=1e6)
CFG5 = dict(hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288, eps=1e-6, rope_theta=1e6)


def bf16_weights(cfg, base):
    H, hq, hkv, d, F = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn"))
    w = dict(gamma1=synth.ones_bf16(H), gamma2=synth.ones_bf16(H),
             w_qkv=synth.normal_bf16(base + 2, ((hq + 2 * hkv) * d, H), 0.02),
             w_o=synth.normal_bf16(base + 3, (H, hq * d), 0.02))
    if F:
        w["w_gate_up"] = synth.normal_bf16(base + 4, (2 * F, H), 0.02)
        w["w_down"] = synth.normal_bf16(base + 6, (H, F), 0.02)
    return w


def int4_weights(cfg, base):
    H, hq, hkv, d, F = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn"))
    return dict(gamma1=synth.ones_bf16(H), gamma2=synth.ones_bf16(H),
                w_qkv=synth.quantize_int4_g32(base + 4, (hq + 2 * hkv) * d, H),
                w_o=synth.quantize_int4_g32(base + 5, H, hq * d),
                w_gate_up=synth.quantize_int4_g32(base + 6, 2 * F, H),
                w_down=synth.quantize_int4_g32(base + 8, H, F))


def to_device_weights(w):
    out = {}
    for k, v in w.items():
        if isinstance(v, tuple):
            out[k] = (torch.from_numpy(v[0]).cuda(), torch.from_numpy(v[1].view(np.int16)).cuda())
        else:
            out[k] = dev(v)
    return out


def make_block(cfg, w):
    bc = bi.BlockConfig(cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn"],
                        cfg["eps"], cfg["rope_theta"], int4=isinstance(w["w_qkv"], tuple))
    return bi.Block(bc, to_device_weights(w))


def stages(ws, lay, cfg, M):
    H, hq, hkv, d, F = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn"))
    widths = dict(n1=H, qkv=(hq + 2 * hkv) * d, q=hq * d, attn=hq * d)
    if F:
        # o and d live only inside the fused residual GEMMs, gate/up inside the SwiGLU GEMM
        widths.update(h=H, n2=H, act=F)
    return {k: bits(bi.stage(ws, lay, k, M, wd)) for k, wd in widths.items()}


def check_fused_stages(x, st, y, gemm, wdev, wref, F, tag=""):
    """The O, gate/up and down projections run fused with their elementwise steps (residual
    add, SwiGLU), so their GEMM outputs are never stored.  Rebuild each with the library's
    unfused GEMM on the same rows (a row's GEMM output does not depend on the other rows),
    check it against the oracle fed the GPU's previous stage, check the step after it against
    the oracle on those bits, and check the fused stage bitwise against the unfused one."""
    o = bits(gemm(dev(st["attn"]), wdev["w_o"]))
    assert_within_tolerance(o, oracle.gemm(st["attn"], wref["w_o"]), "o" + tag)
    assert_bitwise(st["h"], oracle.residual_add(x, o), "h = x + o" + tag)
    assert_within_tolerance(st["n2"], oracle.rmsnorm(st["h"], wref["gamma2"], 1e-6), "n2" + tag)
    gu = gemm(dev(st["n2"]), wdev["w_gate_up"])
    gub = bits(gu)
    assert_within_tolerance(gub, oracle.gemm(st["n2"], wref["w_gate_up"]), "gate/up" + tag)
    assert_within_tolerance(st["act"], oracle.swiglu(gub[:, :F], gub[:, F:]), "swiglu" + tag)
    assert_bitwise(st["act"], bits(bi.swiglu(gu)), "fused gate/up + swiglu vs unfused" + tag)
    d = bits(gemm(dev(st["act"]), wdev["w_down"]))
    assert_within_tolerance(d, oracle.gemm(st["act"], wref["w_down"]), "down" + tag)
    assert_bitwise(y, oracle.residual_add(st["h"], d), "y = h + down" + tag)


# ------------------------------------------------------------- tiny block
def test_tiny_block_invariance_and_parity():
    device()
    cfg = CFG1
    w = bf16_weights(cfg, 100)
    blk = make_block(cfg, w)
    T, H = 128, 256
    xs = [dev(synth.normal_bf16(101 + 10 * i, (T, H))) for i in range(8)]
    kp = torch.zeros((8 * 1024 + 512, 4, 64), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    ncall = [0]

    def backend(reqs, variant):
        # sequence j of the call lives in pool region j (shifted by 512 rows every other
        # call): cache placement must not matter either
        shift = 512 * (ncall[0] % 2)
        ncall[0] += 1
        seqs = [dict(q_len=T, ctx_len=0, kv_base=1024 * j + shift) for j in range(len(reqs))]
        y, _, _ = forward_poisoned(blk, torch.cat([xs[r] for r in reqs]), seqs, kp, vp)
        return split_rows(bits(y), seqs)

    calls = harness.plan(range(8), [3, 8, 5], repeats=10, batch_repeats=3, seed=102)
    rep = harness.run(backend, calls)
    print("tiny block invariance:", rep.summary())
    assert rep.invariant and rep.identical_pct == 100.0, rep.summary()
    # parity on one batch of all 8 in a random order, end to end and stage by stage
    order = list(np.random.default_rng(103).permutation(8))
    seqs = [dict(q_len=T, ctx_len=0, kv_base=1024 * j) for j in range(8)]
    announce("tiny block parity, order", order)
    y, ws, lay = forward_poisoned(blk, torch.cat([xs[i] for i in order]), seqs, kp, vp)
    yb = bits(y)
    M = T * len(order)
    st = stages(ws, lay, cfg, M)
    x_all = np.concatenate([bits(xs[i]) for i in order])
    kpo = np.zeros((8 * 1024, 4, 64), np.uint16); vpo = np.zeros_like(kpo)
    ref = oracle.block_forward(cfg, w, x_all, seqs, kpo, vpo)
    assert_rowwise_norm(yb, ref["y"], "tiny block")
    assert_within_tolerance(st["n1"], oracle.rmsnorm(x_all, w["gamma1"], 1e-6), "stage n1")
    assert_within_tolerance(st["qkv"], oracle.gemm(st["n1"], w["w_qkv"]), "stage qkv")
    q = st["qkv"].reshape(M, 12, 64)
    att = np.concatenate([oracle.attention(q[j * T:(j + 1) * T, :4], q[j * T:(j + 1) * T, 4:8],
                                           q[j * T:(j + 1) * T, 8:], np.arange(T), 1 / 8.0).reshape(T, -1)
                          for j in range(len(order))])
    assert_within_tolerance(st["attn"], att, "stage attention")
    # the O projection is fused with the residual add: rebuild o with the unfused GEMM, check
    # it against the oracle and the fused output bitwise against the oracle's add of those bits
    o = bits(bi.gemm(dev(st["attn"]), dev(w["w_o"])))
    assert_within_tolerance(o, oracle.gemm(st["attn"], w["w_o"]), "stage o")
    assert_bitwise(yb, oracle.residual_add(x_all, o), "stage o + residual")


# ------------------------------------------------------ dense block (4000)
@pytest.fixture(scope="module")
def dense_block():
    device()
    w = bf16_weights(CFG3, 300)
    return w, make_block(CFG3, w)


def run_chunked(blk, x, chunks, kp, vp, base=0):
    ys, s0, last = [], 0, None
    for c in chunks:
        y, ws, lay = forward_poisoned(blk, x[s0:s0 + c], [dict(q_len=c, ctx_len=s0, kv_base=base)], kp, vp)
        ys.append(bits(y))
        last = (ws, lay, s0, c)
        s0 += c
    return np.concatenate(ys), last


def check_dense_stages_sampled(w, wdev, st, x_chunk, y_chunk, kp, vp, s0, rows, tag):
    """Stage-wise parity of sampled rows of one dense-block chunk that starts at position s0
    (each stage's oracle fed the GPU's previous stage; attention over the GPU's cache)."""
    c = len(x_chunk)
    sub = {k: v[rows] for k, v in st.items()}
    assert_within_tolerance(sub["n1"], oracle.rmsnorm(x_chunk[rows], w["gamma1"], 1e-6), "n1" + tag)
    assert_within_tolerance(sub["qkv"], oracle.gemm(sub["n1"], w["w_qkv"]), "qkv" + tag)
    qkv = sub["qkv"].reshape(len(rows), 48, 128)
    pos = s0 + rows
    assert_within_tolerance(sub["q"], oracle.rope(qkv[:, :32], pos, 1e6).reshape(len(rows), -1), "rope q" + tag)
    last = s0 + int(rows.max()) + 1
    kpb, vpb = bits(kp[:last]), bits(vp[:last])
    assert_within_tolerance(kpb[pos], oracle.rope(qkv[:, 32:40], pos, 1e6), "rope k in cache" + tag)
    assert_bitwise(vpb[pos], qkv[:, 40:], "v in cache" + tag)
    att = oracle.attention(sub["q"].reshape(len(rows), 32, 128), kpb, vpb, pos, 1 / math.sqrt(128))
    assert_within_tolerance(sub["attn"], att.reshape(len(rows), -1), "attention" + tag)
    check_fused_stages(x_chunk[rows], sub, y_chunk[rows], lambda a, wt: bi.gemm(a, wt), wdev, w, 9728, tag)


def test_dense_block_parity_stagewise(dense_block):
    w, blk = dense_block
    cfg = CFG3
    T = 600
    x = synth.normal_bf16(301, (4000, 2560))[:T]
    kp = torch.zeros((T, 8, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    announce("dense block parity T=600 as 256 + 344")
    y, (ws, lay, s0, c) = run_chunked(blk, dev(x), [256, 344], kp, vp)
    st = stages(ws, lay, cfg, c)
    xr = x[s0:s0 + c]
    # stage by stage on every row of the second chunk
    check_dense_stages_sampled(w, {k: dev(w[k]) for k in ("w_o", "w_gate_up", "w_down")}, st, xr, y[s0:], kp, vp,
                               s0, np.arange(c), " (T=600, chunk 2)")
    # end to end over both chunks
    kpo = np.zeros((T, 8, 128), np.uint16); vpo = np.zeros_like(kpo)
    ref = oracle.block_forward(cfg, w, x, [dict(q_len=T, ctx_len=0, kv_base=0)], kpo, vpo)
    assert_rowwise_norm(y, ref["y"], "dense block T=600")


def test_dense_block_4000_parity_sampled(dense_block):
    """Stage-wise parity on sampled rows of the 4000-token prompt run as one chunk (the
    folded prefill grid, 16 row tiles per GEMM) and of its last 250-token chunk."""
    w, blk = dense_block
    x = synth.normal_bf16(301, (4000, 2560))
    xd = dev(x)
    wdev = {k: dev(w[k]) for k in ("w_o", "w_gate_up", "w_down")}
    rng = np.random.default_rng(305)
    kp = torch.zeros((4000, 8, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    announce("dense block 4000 as one chunk, sampled stage parity")
    y, (ws, lay, s0, c) = run_chunked(blk, xd, [4000], kp, vp)
    st = stages(ws, lay, CFG3, 4000)
    rows = np.unique(np.concatenate([[0, 1, 31, 32, 63, 64, 127, 255, 2047, 3999], rng.choice(4000, 6, replace=False)]))
    check_dense_stages_sampled(w, wdev, st, x, y, kp, vp, 0, rows, " (4000 chunk)")
    announce("dense block 4000 as 250-token chunks, last chunk sampled stage parity")
    kp2 = torch.zeros_like(kp); vp2 = torch.zeros_like(kp)
    y2, (ws2, lay2, s0, c) = run_chunked(blk, xd, [250] * 16, kp2, vp2)
    assert_bitwise(y2, y, "250-token chunks vs one chunk")
    st2 = stages(ws2, lay2, CFG3, c)
    rows = np.array([0, 1, 100, 249])
    check_dense_stages_sampled(w, wdev, st2, x[s0:], y2[s0:], kp2, vp2, s0, rows, " (last 250 chunk)")


def test_dense_block_4000_chunkings(dense_block):
    """The 4000-token prompt as 1 x 4000, 4 x 1000 and 16 x 250 chunks: the same bits of every
    row and of the KV cache; 10 repeats of each (harness: distinct outputs per chunking)."""
    w, blk = dense_block
    x = dev(synth.normal_bf16(301, (4000, 2560)))
    caches = {}
    kp = torch.zeros((4000, 8, 128), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)

    def backend(reqs, chunk):
        kp.view(torch.int16).fill_(-1); vp.view(torch.int16).fill_(-1)  # NaN cache: stale rows show up
        y, _ = run_chunked(blk, x, [chunk] * (4000 // chunk), kp, vp)
        caches.setdefault(chunk, set()).add(hashlib.sha256(bits(kp).tobytes() + bits(vp).tobytes()).hexdigest())
        return [y]

    calls = [harness.Call(("prompt",), chunk, f"chunks of {chunk} rep {r}") for chunk in (4000, 1000, 250)
             for r in range(10)]
    rep = harness.run(backend, calls, log=announce)
    print("dense block chunkings:", rep.summary())
    assert rep.invariant and rep.observations["prompt"] == 30, rep.summary()
    assert len(set().union(*caches.values())) == 1, "KV cache differs between chunkings or repeats"


# ---------------------------------------------------- int4 mixed step
B_MAX, CAP5 = 256, 8193  # decode requests in the pool; pool rows per request (KV 512..8192, plus the new token)


@pytest.fixture(scope="module")
def int4_block():
    device()
    w = int4_weights(CFG5, 500)
    return w, make_block(CFG5, w)


@pytest.fixture(scope="module")
def int4_pool():
    """256 decode requests with cached lengths ~ U{512..8192} (three of them pinned to 600,
    4200 and 8192 cached keys: 3, 17 and 33 units of 256 after the new token is appended, and
    one at 512: 3 units) and one 2048-token prefill chunk, in one pool of 256 x 8193 + 2048
    rows per K and V (8.6 GB)."""
    lens = synth.uniform_ints(501, B_MAX, 512, 8192)
    lens[:4] = [600, 4200, 8192, 512]
    rows = B_MAX * CAP5 + 2048
    kp = synth.normal_bf16_device(509, (rows, 8, 128))
    vp = synth.normal_bf16_device(510, (rows, 8, 128))
    xdec = synth.normal_bf16(502, (B_MAX, 4096))
    xpre = synth.normal_bf16(503, (2048, 4096))
    return dict(lens=lens, kp=kp, vp=vp, xdec=xdec, xpre=xpre, xdec_d=dev(xdec), xpre_d=dev(xpre),
                pre_base=B_MAX * CAP5)


def int4_seq(pool, r):
    if r == "P":
        return dict(q_len=2048, ctx_len=0, kv_base=pool["pre_base"])
    return dict(q_len=1, ctx_len=int(pool["lens"][r]), kv_base=int(r) * CAP5)


def int4_x(pool, r):
    return pool["xpre_d"] if r == "P" else pool["xdec_d"][r:r + 1]


def test_int4_mixed_step_invariance(int4_block, int4_pool):
    """The benched step's invariance over decode batch 1..256: every decode row bitwise equal
    alone (B = 1, no prefill) and inside mixed steps of B in {1, 2, 8, 64, 256} and a random B
    with the prefill chunk at a random position; the prefill chunk's rows equal alone (1 x 2048
    and 4 x 512) and mixed; 10 repeats of the B = 256 step and of 8 lone requests."""
    w, blk = int4_block
    pool = int4_pool
    kp, vp = pool["kp"], pool["vp"]

    def backend(reqs, variant):
        if variant == "4x512":
            parts = []
            for c in range(4):
                sq = dict(q_len=512, ctx_len=512 * c, kv_base=pool["pre_base"])
                y, _, _ = forward_poisoned(blk, pool["xpre_d"][512 * c:512 * (c + 1)], [sq], kp, vp)
                parts.append(bits(y))
            return [np.concatenate(parts)]
        seqs = [int4_seq(pool, r) for r in reqs]
        y, _, _ = forward_poisoned(blk, torch.cat([int4_x(pool, r) for r in reqs]), seqs, kp, vp)
        return split_rows(bits(y), seqs)

    rng = np.random.default_rng(504)
    calls = [harness.Call((b,), None, f"alone {b}") for b in range(B_MAX)]
    calls += [harness.Call(("P",), None, "prefill alone 1 x 2048"), harness.Call(("P",), "4x512", "prefill alone 4 x 512")]
    for rep in range(1, 10):
        calls += [harness.Call((b,), None, f"alone {b} rep {rep}") for b in (0, 1, 2, 3, 77, 130, 200, 255)]
    full = None
    for B in (1, 2, 8, 64, 256, int(rng.integers(65, 256))):
        idx = [int(b) for b in rng.choice(B_MAX, size=B, replace=False)]
        at = int(rng.integers(0, B + 1))
        ids = tuple(idx[:at] + ["P"] + idx[at:])
        calls.append(harness.Call(ids, None, f"mixed B={B}, prefill at {at}"))
        if B == 256:
            full = ids
            calls.append(harness.Call(ids[::-1], None, "mixed B=256 reversed"))
    calls += [harness.Call(full, None, f"mixed B=256 rep {rep}") for rep in range(1, 10)]
    rep = harness.run(backend, calls, log=lambda m: None if m.startswith("alone") else announce(m))
    print("int4 mixed step invariance:", rep.summary())
    assert rep.invariant and rep.identical_pct == 100.0, rep.summary()
    assert len(rep.distinct) == B_MAX + 1 and rep.observations["P"] >= 2 + 6 + 10


def test_int4_mixed_step_parity_sampled(int4_block, int4_pool):
    """Stage-wise parity of sampled rows of the benched B = 256 mixed step: decode requests of
    3, 17 and 33 units (and 3 at the 512-key boundary), random decode rows and prefill rows."""
    w, blk = int4_block
    pool = int4_pool
    kp, vp = pool["kp"], pool["vp"]
    order = [int(b) for b in np.random.default_rng(514).permutation(B_MAX)]
    at = 100
    ids = order[:at] + ["P"] + order[at:]
    seqs = [int4_seq(pool, r) for r in ids]
    x = np.concatenate([pool["xpre"] if r == "P" else pool["xdec"][r:r + 1] for r in ids])
    announce("int4 mixed step B=256 parity")
    y, ws, lay = forward_poisoned(blk, dev(x), seqs, kp, vp)
    M = B_MAX + 2048
    st = stages(ws, lay, CFG5, M)
    yb = bits(y)
    row_of = {r: (order.index(r) if order.index(r) < at else order.index(r) + 2048) for r in range(B_MAX)}
    dec = [0, 1, 2, 3] + [int(b) for b in np.random.default_rng(515).choice(np.arange(4, B_MAX), 4, replace=False)]
    prow = np.array([0, 1, 63, 64, 511, 2047])
    rows = np.array([row_of[b] for b in dec] + list(at + prow))
    deq = {k: oracle.dequant_int4_g32(*w[k]) for k in ("w_qkv", "w_o", "w_gate_up", "w_down")}
    assert_within_tolerance(st["n1"][rows], oracle.rmsnorm(x[rows], w["gamma1"], 1e-6), "n1")
    assert_within_tolerance(st["qkv"][rows], oracle.gemm(st["n1"][rows], deq["w_qkv"]), "qkv (int4)")
    q4 = {k: (torch.from_numpy(w[k][0]).cuda(), torch.from_numpy(w[k][1].view(np.int16)).cuda())
          for k in ("w_o", "w_gate_up", "w_down")}
    w4 = lambda a, wt: bi.gemm_w4(a, *wt)
    sub = {k: v[rows] for k, v in st.items()}
    check_fused_stages(x[rows], sub, yb[rows], w4, q4, dict(deq, gamma2=w["gamma2"]), 12288, " (int4)")
    # RoPE of the new tokens, and decode attention over the GPU's own cache contents
    q = st["q"].reshape(M, 32, 128)
    qkv = st["qkv"].reshape(M, 48, 128)
    for b in dec:
        r, L = row_of[b], int(pool["lens"][b]) + 1
        base = b * CAP5
        kb, vb = bits(kp[base:base + L]), bits(vp[base:base + L])
        p = np.array([L - 1])
        assert_within_tolerance(q[r:r + 1], oracle.rope(qkv[r:r + 1, :32], p, 1e6), f"rope q b={b}")
        assert_within_tolerance(kb[L - 1:], oracle.rope(qkv[r:r + 1, 32:40], p, 1e6), f"rope k b={b}")
        assert_bitwise(vb[L - 1:], qkv[r:r + 1, 40:], f"v appended b={b}")
        ref = oracle.decode_attention(q[r], kb, vb, 1 / math.sqrt(128))
        assert_within_tolerance(st["attn"][r], ref.reshape(-1), f"decode attention b={b} ({(L + 255) // 256} units)")
    kb, vb = bits(kp[pool["pre_base"]:pool["pre_base"] + 2048]), bits(vp[pool["pre_base"]:pool["pre_base"] + 2048])
    ref = oracle.attention(q[at + prow], kb, vb, prow, 1 / math.sqrt(128))
    assert_within_tolerance(st["attn"][at + prow], ref.reshape(len(prow), -1), "prefill attention rows")


# --------------------------------------- int4 block over the paged int8 KV cache
B_Q8 = 64
PAGE = 64  # rows per page of the int8 cache


@pytest.fixture(scope="module")
def q8_setup(int4_block, int4_pool):
    """The int4 block on a quantised, paged cache: the first 64 decode requests of the pool
    above and the prefill chunk, their pages scattered over the pool in random order (some
    pages unused), the decode requests' cached context quantised into their pages."""
    w, _ = int4_block
    lens = int4_pool["lens"][:B_Q8]
    rng = np.random.default_rng(530)
    npg = [(int(L) + 1 + PAGE - 1) // PAGE for L in lens] + [2048 // PAGE, 300 // PAGE + 1]
    total = int(sum(npg))
    perm = rng.permutation(total + 9)[:total].astype(np.int32)
    entries = np.concatenate([[0], np.cumsum(npg)[:-1]]).astype(np.int64)
    pool = bi.KvPoolQ8(total + 9, 8, 128, page_table=torch.from_numpy(perm).cuda())
    rows = np.concatenate([perm[entries[b] + np.arange(L) // PAGE].astype(np.int64) * PAGE + np.arange(L) % PAGE
                           for b, L in enumerate(lens)])
    k = synth.normal_bf16_device(531, (len(rows), 8, 128))
    v = synth.normal_bf16_device(532, (len(rows), 8, 128))
    bi.kv_append_q8(pool, k, v, torch.from_numpy(rows).cuda())
    torch.cuda.synchronize()
    del k, v
    cfg = dict(CFG5)
    bc = bi.BlockConfig(cfg["hidden"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["ffn"], cfg["eps"],
                        cfg["rope_theta"], int4=True, decode_prefill_order=True, kv_q8=True)
    blk = bi.Block(bc, to_device_weights(w))
    return dict(pool=pool, perm=perm, entries=entries, lens=lens, blk=blk)


def q8_seq(q8, r):
    if r == "P":
        return dict(q_len=2048, ctx_len=0, kv_base=int(q8["entries"][B_Q8]))
    return dict(q_len=1, ctx_len=int(q8["lens"][r]), kv_base=int(q8["entries"][r]))


def q8_rows(q8, r, L):
    """Pool rows of positions 0 .. L - 1 of request r."""
    e = int(q8["entries"][B_Q8 if r == "P" else (B_Q8 + 1 if r == "S" else r)])
    p = np.arange(L)
    return q8["perm"][e + p // PAGE].astype(np.int64) * PAGE + p % PAGE


def test_int4_block_q8_cache_invariance(q8_setup, int4_pool):
    """Over the paged int8 cache: each decode row bitwise equal alone and in mixed steps of
    B in {1, 8, 64} at any position; the prefill chunk as 1 x 2048 and 4 x 512; repeats; and
    a token's bits the same prefilled or decoded (a 300-token prompt whole, vs 298 tokens
    then two decodes)."""
    q8 = q8_setup
    blk, pool = q8["blk"], q8["pool"]
    xpre_d, xdec_d = int4_pool["xpre_d"], int4_pool["xdec_d"]

    def backend(reqs, variant):
        if variant == "4x512":
            parts = []
            for c in range(4):
                sq = dict(q_len=512, ctx_len=512 * c, kv_base=int(q8["entries"][B_Q8]))
                y, _, _ = forward_poisoned(blk, xpre_d[512 * c:512 * (c + 1)], [sq], pool, None)
                parts.append(bits(y))
            return [np.concatenate(parts)]
        seqs = [q8_seq(q8, r) for r in reqs]
        x = torch.cat([xpre_d if r == "P" else xdec_d[r:r + 1] for r in reqs])
        y, _, _ = forward_poisoned(blk, x, seqs, pool, None)
        return split_rows(bits(y), seqs)

    rng = np.random.default_rng(533)
    calls = [harness.Call((b,), None, f"alone {b}") for b in range(B_Q8)]
    calls += [harness.Call(("P",), None, "prefill 1 x 2048"), harness.Call(("P",), "4x512", "prefill 4 x 512")]
    for B in (1, 8, 64):
        idx = [int(b) for b in rng.choice(B_Q8, size=B, replace=False)]
        at = int(rng.integers(0, B + 1))
        ids = tuple(idx[:at] + ["P"] + idx[at:])
        calls += [harness.Call(ids, None, f"q8 mixed B={B} rep {r}") for r in range(3)]
        calls.append(harness.Call(ids[::-1], None, f"q8 mixed B={B} reversed"))
    rep = harness.run(backend, calls, log=lambda m: None if m.startswith("alone") else announce(m))
    print("int4 block, paged int8 cache:", rep.summary())
    assert rep.invariant and rep.identical_pct == 100.0, rep.summary()
    # decode bits = prefill bits through the quantised cache
    xs = dev(synth.normal_bf16(534, (300, 4096)))
    e = int(q8["entries"][B_Q8 + 1])
    announce("q8 block: 300-token prompt whole vs 298 + two decodes")
    whole, _, _ = forward_poisoned(blk, xs, [dict(q_len=300, ctx_len=0, kv_base=e)], pool, None)
    whole = bits(whole)
    part, _, _ = forward_poisoned(blk, xs[:298], [dict(q_len=298, ctx_len=0, kv_base=e)], pool, None)
    rows = [bits(part)]
    for t in (298, 299):
        y, _, _ = forward_poisoned(blk, xs[t:t + 1], [dict(q_len=1, ctx_len=t, kv_base=e)], pool, None)
        rows.append(bits(y))
    assert_bitwise(np.concatenate(rows), whole, "q8 block: prefilled vs decoded rows")


def test_int4_block_q8_cache_parity(q8_setup, int4_block, int4_pool):
    """Stage-wise parity of a B = 64 mixed step over the paged int8 cache: the rotated keys and
    values against the oracle, the int8 codes and scales stored for them bitwise against the
    oracle's quantisation of those bits, attention against the oracle on the dequantised pages,
    then the fused projections, on sampled decode and prefill rows."""
    q8 = q8_setup
    w, _ = int4_block
    blk, pool = q8["blk"], q8["pool"]
    order = [int(b) for b in np.random.default_rng(535).permutation(B_Q8)]
    at = 20
    ids = order[:at] + ["P"] + order[at:]
    seqs = [q8_seq(q8, r) for r in ids]
    x = np.concatenate([int4_pool["xpre"] if r == "P" else int4_pool["xdec"][r:r + 1] for r in ids])
    announce("q8 block B=64 mixed step parity")
    y, ws, lay = forward_poisoned(blk, dev(x), seqs, pool, None)
    M = B_Q8 + 2048
    st = stages(ws, lay, CFG5, M)
    yb = bits(y)
    kv_new = bits(ws[lay.kv_new:lay.kv_new + 2 * M * 8 * 128 * 2].view(torch.bfloat16)).reshape(2, M, 8, 128)
    row_of = {r: (order.index(r) if order.index(r) < at else order.index(r) + 2048) for r in range(B_Q8)}
    dec = [0, 1, 2, 3] + [int(b) for b in np.random.default_rng(536).choice(np.arange(4, B_Q8), 3, replace=False)]
    prow = np.array([0, 1, 63, 64, 1000, 2047])
    rows = np.array([row_of[b] for b in dec] + list(at + prow))
    pos = np.array([int(q8["lens"][b]) for b in dec] + list(prow))
    qkv = st["qkv"].reshape(M, 48, 128)
    assert_within_tolerance(kv_new[0][rows], oracle.rope(qkv[rows, 32:40], pos, 1e6), "rotated keys")
    assert_bitwise(kv_new[1][rows], qkv[rows, 40:], "values")
    # codes and scales stored for the step's tokens, bitwise against the oracle's quantisation
    kq, ks = KV.quantize(kv_new[0][rows])
    vq, vs = KV.quantize(kv_new[1][rows])
    dst = np.array([q8_rows(q8, b, int(q8["lens"][b]) + 1)[-1] for b in dec] +
                   list(q8_rows(q8, "P", 2048)[prow]))
    dst_d = torch.from_numpy(dst).cuda()
    assert_bitwise(pool.k[dst_d].cpu().numpy(), kq, "stored key codes")
    assert_bitwise(pool.v[dst_d].cpu().numpy(), vq, "stored value codes")
    assert_bitwise(pool.ks[dst_d].cpu().numpy().view(np.uint32), ks.view(np.uint32), "stored key scales")
    assert_bitwise(pool.vs[dst_d].cpu().numpy().view(np.uint32), vs.view(np.uint32), "stored value scales")
    # attention over the dequantised pages
    q = st["q"].reshape(M, 32, 128)

    def deq(r, L):
        pr = torch.from_numpy(q8_rows(q8, r, L)).cuda()
        return (KV.dequantize(pool.k[pr].cpu().numpy(), pool.ks[pr].cpu().numpy()),
                KV.dequantize(pool.v[pr].cpu().numpy(), pool.vs[pr].cpu().numpy()))

    for b in dec:
        r, L = row_of[b], int(q8["lens"][b]) + 1
        kb, vb = deq(b, L)
        ref = oracle.decode_attention(q[r], kb, vb, 1 / math.sqrt(128))
        assert_within_tolerance(st["attn"][r], ref.reshape(-1), f"q8 decode attention b={b}")
    kb, vb = deq("P", 2048)
    ref = oracle.attention(q[at + prow], kb, vb, prow, 1 / math.sqrt(128))
    assert_within_tolerance(st["attn"][at + prow], ref.reshape(len(prow), -1), "q8 prefill attention rows")
    # the projections after attention
    deqw = {k: oracle.dequant_int4_g32(*w[k]) for k in ("w_o", "w_gate_up", "w_down")}
    q4 = {k: (torch.from_numpy(w[k][0]).cuda(), torch.from_numpy(w[k][1].view(np.int16)).cuda())
          for k in ("w_o", "w_gate_up", "w_down")}
    sub = {k: v[rows] for k, v in st.items()}
    check_fused_stages(x[rows], sub, yb[rows], lambda a, wt: bi.gemm_w4(a, *wt), q4, dict(deqw, gamma2=w["gamma2"]),
                       12288, " (q8 cache)")
