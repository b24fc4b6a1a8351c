"""Pins for the oracle's decoder block (a composition of the pinned parts).

Structural special cases fix the wiring: zero output projections make the
block the identity; with identity value/output weights a one-token sequence
gives h = x + RMSNorm(x); appended keys/values land at absolute positions;
chunked prefill and batching give the same bits as one whole pass alone; int4
weights give the same bits as their de-quantised bf16 weights.
"""
import numpy as np

from oracle import block_forward, dequant_int4_g32, residual_add, rmsnorm
from invariant_deterministic_amd import synth

CFG1 = dict(hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=0, eps=1e-6, rope_theta=0.0)
CFG_SMALL = dict(hidden=128, n_q_heads=4, n_kv_heads=2, head_dim=32, ffn=96, eps=1e-6, rope_theta=1e4)


def weights(cfg, seed=0):
    H, hq, hkv, d, F = (cfg[k] for k in ("hidden", "n_q_heads", "n_kv_heads", "head_dim", "ffn"))
    w = dict(gamma1=synth.ones_bf16(H), gamma2=synth.ones_bf16(H),
             w_qkv=synth.normal_bf16(seed + 1, ((hq + 2 * hkv) * d, H), 0.02),
             w_o=synth.normal_bf16(seed + 2, (H, hq * d), 0.02))
    if F:
        w["w_gate_up"] = synth.normal_bf16(seed + 3, (2 * F, H), 0.02)
        w["w_down"] = synth.normal_bf16(seed + 4, (H, F), 0.02)
    return w


def pools(cfg, rows):
    shape = (rows, cfg["n_kv_heads"], cfg["head_dim"])
    return np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)


def run(cfg, w, x, seqs, rows=512):
    kp, vp = pools(cfg, rows)
    st = block_forward(cfg, w, x, seqs, kp, vp)
    return st, kp, vp


def test_zero_projections_make_identity():
    cfg = CFG_SMALL
    w = weights(cfg)
    w["w_o"] = np.zeros_like(w["w_o"])
    w["w_down"] = np.zeros_like(w["w_down"])
    x = synth.normal_bf16(1, (20, cfg["hidden"]))
    st, _, _ = run(cfg, w, x, [dict(q_len=20, ctx_len=0, kv_base=0)])
    np.testing.assert_array_equal(st["y"], x)


def test_identity_value_path_one_token():
    cfg = CFG1
    H = cfg["hidden"]
    w = weights(cfg)
    wq = w["w_qkv"].copy()
    wq[2 * H:3 * H] = synth.to_bf16_bits(np.eye(H, dtype=np.float32))  # v rows = identity
    w["w_qkv"] = wq
    w["w_o"] = synth.to_bf16_bits(np.eye(H, dtype=np.float32))
    x = synth.normal_bf16(2, (3, H))
    seqs = [dict(q_len=1, ctx_len=0, kv_base=64 * i) for i in range(3)]
    st, _, _ = run(cfg, w, x, seqs)
    n1 = rmsnorm(x, w["gamma1"], cfg["eps"])
    np.testing.assert_array_equal(st["attn"], n1)
    np.testing.assert_array_equal(st["y"], residual_add(x, n1))


def test_kv_append_at_absolute_positions():
    cfg = CFG_SMALL
    w = weights(cfg)
    x = synth.normal_bf16(3, (7, cfg["hidden"]))
    kp, vp = pools(cfg, 256)
    kp[100:105] = synth.normal_bf16(4, (5,) + kp.shape[1:])  # cached context
    vp[100:105] = synth.normal_bf16(5, (5,) + vp.shape[1:])
    st = block_forward(cfg, w, x, [dict(q_len=7, ctx_len=5, kv_base=100)], kp, vp)
    M = 7
    np.testing.assert_array_equal(kp[105:112].reshape(M, -1), st["k"])
    np.testing.assert_array_equal(vp[105:112].reshape(M, -1), st["v"])
    assert np.all(kp[112:] == 0) and np.all(kp[:100] == 0)


def test_chunked_prefill_equals_whole():
    cfg = CFG_SMALL
    w = weights(cfg)
    T = 48
    x = synth.normal_bf16(6, (T, cfg["hidden"]))
    whole, kw, vw = run(cfg, w, x, [dict(q_len=T, ctx_len=0, kv_base=0)])
    kp, vp = pools(cfg, 512)
    ys = []
    for c0 in range(0, T, 13):
        n = min(13, T - c0)
        st = block_forward(cfg, w, x[c0:c0 + n], [dict(q_len=n, ctx_len=c0, kv_base=0)], kp, vp)
        ys.append(st["y"])
    np.testing.assert_array_equal(np.concatenate(ys), whole["y"])
    np.testing.assert_array_equal(kp, kw)
    np.testing.assert_array_equal(vp, vw)


def test_batched_equals_alone():
    cfg = CFG_SMALL
    w = weights(cfg)
    lens = [5, 1, 9, 1]
    ctx = [0, 6, 3, 11]
    xs = [synth.normal_bf16(10 + i, (n, cfg["hidden"])) for i, n in enumerate(lens)]
    cache_k = [synth.normal_bf16(20 + i, (c, cfg["n_kv_heads"], cfg["head_dim"])) for i, c in enumerate(ctx)]
    cache_v = [synth.normal_bf16(30 + i, (c, cfg["n_kv_heads"], cfg["head_dim"])) for i, c in enumerate(ctx)]
    alone = []
    for i in range(4):
        kp, vp = pools(cfg, 64)
        kp[:ctx[i]] = cache_k[i]; vp[:ctx[i]] = cache_v[i]
        alone.append(block_forward(cfg, w, xs[i], [dict(q_len=lens[i], ctx_len=ctx[i], kv_base=0)], kp, vp)["y"])
    kp, vp = pools(cfg, 256)
    seqs = []
    for i in range(4):
        kp[64 * i:64 * i + ctx[i]] = cache_k[i]; vp[64 * i:64 * i + ctx[i]] = cache_v[i]
        seqs.append(dict(q_len=lens[i], ctx_len=ctx[i], kv_base=64 * i))
    y = block_forward(cfg, w, np.concatenate(xs), seqs, kp, vp)["y"]
    np.testing.assert_array_equal(y, np.concatenate(alone))


def test_int4_block_equals_dequantised_bf16_block():
    cfg = CFG_SMALL
    H, F = cfg["hidden"], cfg["ffn"]
    hq, hkv, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    q4 = dict(w_qkv=synth.quantize_int4_g32(41, (hq + 2 * hkv) * d, H),
              w_o=synth.quantize_int4_g32(42, H, hq * d),
              w_gate_up=synth.quantize_int4_g32(43, 2 * F, H),
              w_down=synth.quantize_int4_g32(44, H, F))
    w4 = dict(gamma1=synth.ones_bf16(H), gamma2=synth.ones_bf16(H), **q4)
    wb = dict(gamma1=synth.ones_bf16(H), gamma2=synth.ones_bf16(H),
              **{k: dequant_int4_g32(*v) for k, v in q4.items()})
    x = synth.normal_bf16(7, (9, H))
    s = [dict(q_len=9, ctx_len=0, kv_base=0)]
    np.testing.assert_array_equal(run(cfg, w4, x, s)[0]["y"], run(cfg, wb, x, s)[0]["y"])
