"""GPU tests of bi_block_forward: parity against the oracle (end-to-end and
stage by stage) and bitwise invariance of every request's rows across batch
size, batch position, prefill chunking and repeats.

Shapes: the tiny block (hidden 256, 4 heads of 64, no RoPE, no FFN), the dense
Qwen3-4B-shaped block (hidden 2560, 32/8 heads of 128, RoPE 1e6, SwiGLU 9728)
and the int4 block (hidden 4096, FFN 12288) on a mixed decode + prefill step.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import bi, synth
from tests.gpu_util import announce, assert_bitwise, bits, dev, device
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
    xs = [synth.normal_bf16(101 + 10 * i, (T, H)) for i in range(8)]
    kp = torch.zeros((8 * 1024, 4, 64), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    # alone, each sequence at its own pool region
    alone = []
    for i in range(8):
        announce("tiny block alone", i)
        y, ws, lay = blk.forward(dev(xs[i]), [dict(q_len=T, ctx_len=0, kv_base=1024 * i)], kp, vp)
        alone.append(bits(y))
    # batched: B = 3 and B = 8, rotations and a random permutation, other pool regions
    rng = np.random.default_rng(102)
    orders = [list(range(3)), [1, 2, 0], [2, 0, 1], list(range(8)), list(rng.permutation(8)), [7, 6, 5, 4, 3, 2, 1, 0]]
    for order in orders:
        for rep in range(2):
            announce("tiny block batch", order, rep)
            seqs = [dict(q_len=T, ctx_len=0, kv_base=1024 * j + 512) for j in range(len(order))]
            y, ws, lay = blk.forward(dev(np.concatenate([xs[i] for i in order])), seqs, kp, vp)
            yb = bits(y)
            for j, i in enumerate(order):
                assert_bitwise(yb[j * T:(j + 1) * T], alone[i], f"tiny block seq {i} at position {j} of {len(order)}")
    # parity on the last batch, end to end and stage by stage
    M = T * len(order)
    st = stages(ws, lay, cfg, M)
    x_all = np.concatenate([xs[i] for i in order])
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
        y, ws, lay = blk.forward(x[s0:s0 + c], [dict(q_len=c, ctx_len=s0, kv_base=base)], kp, vp)
        ys.append(bits(y))
        last = (ws, lay, s0, c)
        s0 += c
    return np.concatenate(ys), last


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
    # stage by stage on the second chunk (each stage fed the GPU's previous stage)
    assert_within_tolerance(st["n1"], oracle.rmsnorm(xr, w["gamma1"], 1e-6), "n1")
    assert_within_tolerance(st["qkv"], oracle.gemm(st["n1"], w["w_qkv"]), "qkv")
    qkv = st["qkv"].reshape(c, 48, 128)
    pos = np.arange(s0, s0 + c)
    assert_within_tolerance(st["q"], oracle.rope(qkv[:, :32], pos, 1e6).reshape(c, -1), "rope q")
    kpb, vpb = bits(kp), bits(vp)
    assert_within_tolerance(kpb[s0:s0 + c], oracle.rope(qkv[:, 32:40], pos, 1e6), "rope k in cache")
    assert_bitwise(vpb[s0:s0 + c], qkv[:, 40:], "v in cache")
    att = oracle.attention(st["q"].reshape(c, 32, 128), kpb[:s0 + c], vpb[:s0 + c], pos, 1 / math.sqrt(128))
    assert_within_tolerance(st["attn"], att.reshape(c, -1), "attention")
    bf = lambda a, wt: bi.gemm(a, wt)
    check_fused_stages(xr, st, y[s0:], bf, {k: dev(w[k]) for k in ("w_o", "w_gate_up", "w_down")}, w, 9728)
    # end to end over both chunks
    kpo = np.zeros((T, 8, 128), np.uint16); vpo = np.zeros_like(kpo)
    ref = oracle.block_forward(cfg, w, x, [dict(q_len=T, ctx_len=0, kv_base=0)], kpo, vpo)
    assert_rowwise_norm(y, ref["y"], "dense block T=600")


def test_dense_block_4000_chunkings(dense_block):
    w, blk = dense_block
    x = dev(synth.normal_bf16(301, (4000, 2560)))
    outs, caches = {}, {}
    for chunk in (4000, 1000, 250):
        announce("dense block 4000 tokens in chunks of", chunk)
        kp = torch.zeros((4000, 8, 128), dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        outs[chunk], _ = run_chunked(blk, x, [chunk] * (4000 // chunk), kp, vp)
        caches[chunk] = (bits(kp), bits(vp))
    for chunk in (1000, 250):
        assert_bitwise(outs[chunk], outs[4000], f"block output, chunks of {chunk} vs 4000")
        assert_bitwise(caches[chunk][0], caches[4000][0], f"K cache, chunks of {chunk}")
        assert_bitwise(caches[chunk][1], caches[4000][1], f"V cache, chunks of {chunk}")
    for rep in range(3):
        kp = torch.zeros((4000, 8, 128), dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        y, _ = run_chunked(blk, x, [4000], kp, vp)
        assert_bitwise(y, outs[4000], "block repeat")


# ---------------------------------------------------- int4 mixed step
@pytest.fixture(scope="module")
def int4_block():
    device()
    w = int4_weights(CFG5, 500)
    return w, make_block(CFG5, w)


def test_int4_mixed_step_invariance(int4_block):
    w, blk = int4_block
    H = 4096
    Bmax = 64
    lens = synth.uniform_ints(501, Bmax, 512, 8192)
    xdec = synth.normal_bf16(502, (Bmax, H))
    xpre = synth.normal_bf16(503, (2048, H))
    cap = 8192 + 1
    rows = Bmax * cap + 2048
    kp = synth.normal_bf16_device(509, (rows, 8, 128))
    vp = synth.normal_bf16_device(510, (rows, 8, 128))
    pre_base = Bmax * cap
    xdec_d, xpre_d = dev(xdec), dev(xpre)
    alone = []
    for b in range(Bmax):
        y, _, _ = blk.forward(xdec_d[b:b + 1], [dict(q_len=1, ctx_len=int(lens[b]), kv_base=b * cap)], kp, vp)
        alone.append(bits(y)[0])
    announce("int4 prefill alone 1 x 2048")
    y, _, _ = blk.forward(xpre_d, [dict(q_len=2048, ctx_len=0, kv_base=pre_base)], kp, vp)
    pre_alone = bits(y)
    announce("int4 prefill alone 4 x 512")
    parts = []
    for c in range(4):
        y, _, _ = blk.forward(xpre_d[512 * c:512 * (c + 1)], [dict(q_len=512, ctx_len=512 * c, kv_base=pre_base)], kp, vp)
        parts.append(bits(y))
    assert_bitwise(np.concatenate(parts), pre_alone, "int4 prefill 4 x 512 vs 1 x 2048")
    rng = np.random.default_rng(504)
    for B in (1, 2, 8, 64, int(rng.integers(3, 64))):
        idx = rng.choice(Bmax, size=B, replace=False)
        announce("int4 mixed step B =", B)
        seqs = [dict(q_len=1, ctx_len=int(lens[b]), kv_base=int(b) * cap) for b in idx]
        at = int(rng.integers(0, B + 1))  # where the prefill chunk sits in the batch
        seqs.insert(at, dict(q_len=2048, ctx_len=0, kv_base=pre_base))
        xs = [xdec[b:b + 1] for b in idx]
        xs.insert(at, xpre)
        y, ws, lay = blk.forward(dev(np.concatenate(xs)), seqs, kp, vp)
        yb = bits(y)
        row = 0
        for s in seqs:
            if s["q_len"] == 1:
                b = s["kv_base"] // cap
                assert_bitwise(yb[row], alone[b], f"decode request {b} in mixed step B={B}")
            else:
                assert_bitwise(yb[row:row + 2048], pre_alone, f"prefill chunk in mixed step B={B}")
            row += s["q_len"]


def test_int4_mixed_step_parity_sampled(int4_block):
    """Stage-wise parity of sampled rows of a B = 16 mixed step."""
    w, blk = int4_block
    H, B = 4096, 16
    lens = synth.uniform_ints(511, B, 512, 8192)
    cap = 8193
    kp = synth.normal_bf16_device(519, (B * cap + 2048, 8, 128))
    vp = synth.normal_bf16_device(520, (B * cap + 2048, 8, 128))
    seqs = [dict(q_len=1, ctx_len=int(lens[b]), kv_base=b * cap) for b in range(B)]
    seqs.append(dict(q_len=2048, ctx_len=0, kv_base=B * cap))
    x = np.concatenate([synth.normal_bf16(512, (B, H)), synth.normal_bf16(513, (2048, H))])
    announce("int4 mixed step parity")
    y, ws, lay = blk.forward(dev(x), seqs, kp, vp)
    M = B + 2048
    st = stages(ws, lay, CFG5, M)
    yb = bits(y)
    rows = np.array([0, 5, 15, 16, 17, 100, 1000, M - 1])
    deq = {k: oracle.dequant_int4_g32(*w[k]) for k in ("w_qkv", "w_o", "w_gate_up", "w_down")}
    assert_within_tolerance(st["n1"][rows], oracle.rmsnorm(x[rows], w["gamma1"], 1e-6), "n1")
    assert_within_tolerance(st["qkv"][rows], oracle.gemm(st["n1"][rows], deq["w_qkv"]), "qkv (int4)")
    q4 = {k: (torch.from_numpy(w[k][0]).cuda(), torch.from_numpy(w[k][1].view(np.int16)).cuda())
          for k in ("w_o", "w_gate_up", "w_down")}
    w4 = lambda a, wt: bi.gemm_w4(a, *wt)
    sub = {k: v[rows] for k, v in st.items()}
    check_fused_stages(x[rows], sub, yb[rows], w4, q4, dict(deq, gamma2=w["gamma2"]), 12288, " (int4)")
    # attention of decode rows 0, 5 and prefill rows, against the GPU's own cache contents
    kpb_rows = lambda b, L: (bits(kp[b * cap:b * cap + L]), bits(vp[b * cap:b * cap + L]))
    q = st["q"].reshape(M, 32, 128)
    for b in (0, 5, 15):
        L = int(lens[b]) + 1
        kb, vb = kpb_rows(b, L)
        ref = oracle.decode_attention(q[b], kb, vb, 1 / math.sqrt(128))
        assert_within_tolerance(st["attn"][b], ref.reshape(-1), f"decode attention b={b}")
    kb, vb = kpb_rows(B, 2048)
    prow = np.array([0, 1, 511, 2047])
    ref = oracle.attention(q[B + prow], kb, vb, prow, 1 / math.sqrt(128))
    assert_within_tolerance(st["attn"][B + prow], ref.reshape(len(prow), -1), "prefill attention rows")
