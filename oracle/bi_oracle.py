"""CPU oracle for the batch-invariant transformer forward path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check and the bench's
CPU-baseline leg use it.  It shares no code, table or helper with the HIP
library; the two meet only through the seeded input arrays.

What it computes.  The pages ("Deterministic and bit-exact inference", M-0002
record, field ``technical``, the Invariance route; same record, body section
"How it works") say batch-invariant kernels fix the reduction order of every
output element, for RMSNorm, matrix multiplication and attention, the last with
a fixed split *size* of the key/value dimension.  Fixing an order does not
change what is being computed: each operation still has its plain
mathematical definition.  This oracle therefore writes those definitions out,
evaluated in float64, with a single round-to-nearest-even to bf16 at every
point where the library hands a bf16 tensor from one kernel to the next.  It
never emulates any particular summation order.

Precision.  Products of two bf16 values are exact in float64; the sums are
float64 (library matmul / numpy sums may reorder them, which moves the result
by ~1e-16 relative, far below one bf16 ulp).  float64 -> bf16 rounding is done
directly (``bf16_round``), never through float32.

Parity status.  Every function here is pinned by CPU tests against closed
forms, exact integer arithmetic, library routines or brute force (see
tests/test_oracle_*.py).  ``block_forward`` is a composition of the pinned
parts; its end-to-end bits are pinned only through those parts plus the
structural special cases tested for it.

Layouts.  All bf16 tensors are numpy uint16 arrays of raw bit patterns,
row-major.  fp16 scales are uint16 bit patterns as well.
"""
from __future__ import annotations

import numpy as np

BF16_MAX_EXP = 128  # |x| >= 2**128 rounds to infinity


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------

def bf16_decode(bits) -> np.ndarray:
    """Exact float64 value of bf16 bit patterns (bf16 is the top half of fp32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f16_decode(bits) -> np.ndarray:
    """Exact float64 value of IEEE binary16 bit patterns."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_round(x) -> np.ndarray:
    """float64 -> bf16 bits, round to nearest, ties to even, in one step.

    bf16 keeps 8 significant bits and fp32's exponent range.  For a value
    with |x| in [2**(e-1), 2**e) the spacing of bf16 numbers is 2**(e-8);
    below the normal range the spacing stays at the subnormal quantum 2**-133.
    Rounding x to a multiple of that spacing with ties to even (``np.rint``)
    is IEEE round-to-nearest-even.  Results of magnitude >= 2**128 overflow
    to infinity; NaN maps to the quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e.astype(np.int64) - 8, -133)
    with np.errstate(invalid="ignore", over="ignore"):
        r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
        r = np.where(np.abs(r) >= 2.0 ** BF16_MAX_EXP, np.copysign(np.inf, x), r)
    # r is now exactly representable in bf16, hence in float32: the float32
    # conversion is exact and its top 16 bits are the bf16 pattern.
    out = (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    out = np.where(np.isnan(x), np.uint16(0x7FC0), out)
    return out.astype(np.uint16)


# ---------------------------------------------------------------------------
# RMSNorm  ("How it works": RMSNorm is one of the three operations made
# batch-invariant; the definition is the standard root-mean-square norm)
# ---------------------------------------------------------------------------

def rmsnorm(x_bits, gamma_bits, eps) -> np.ndarray:
    """y[r, j] = bf16( x[r, j] / sqrt(mean_j x[r, j]**2 + eps) * gamma[j] ).

    ``eps`` is the float32 value the library receives, taken exactly.
    """
    x = bf16_decode(x_bits)
    g = bf16_decode(gamma_bits)
    h = x.shape[-1]
    eps64 = float(np.float32(eps))
    ms = np.sum(x * x, axis=-1, keepdims=True) / h
    r = 1.0 / np.sqrt(ms + eps64)
    return bf16_round(x * r * g)


# ---------------------------------------------------------------------------
# matrix multiplication ("technical": matrix multiplication made invariant)
# ---------------------------------------------------------------------------

def gemm(a_bits, w_bits) -> np.ndarray:
    """C = bf16(A @ W^T) with A[M, K], W[N, K]; the K-sum is taken in float64."""
    a = bf16_decode(a_bits)
    w = bf16_decode(w_bits)
    return bf16_round(a @ w.T)


def int4_codes(wq) -> np.ndarray:
    """Signed int4 codes [N, K] from packed bytes [N, K/2] (element 2i = low nibble)."""
    b = np.asarray(wq, dtype=np.uint8)
    lo = (b & 0x0F).astype(np.int64)
    hi = (b >> 4).astype(np.int64)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    n, half = b.shape
    q = np.empty((n, 2 * half), dtype=np.int64)
    q[:, 0::2] = lo
    q[:, 1::2] = hi
    return q


def dequant_int4_g32(wq, ws_bits) -> np.ndarray:
    """bf16 weight W[j, k] = bf16(code[j, k] * scale[j, k // 32]).

    De-quantisation is a plain per-element product with no accumulation at
    all, which is what keeps it free of the atomic additions that the
    "Residual nondeterminism" limitation of the M-0002 record warns about.
    """
    q = int4_codes(wq).astype(np.float64)
    s = f16_decode(ws_bits)
    s_full = np.repeat(s, 32, axis=1)
    return bf16_round(q * s_full)


def gemm_w4(a_bits, wq, ws_bits) -> np.ndarray:
    """C = bf16(A @ dequant(Wq, Ws)^T)."""
    return gemm(a_bits, dequant_int4_g32(wq, ws_bits))


# ---------------------------------------------------------------------------
# rotary position embedding (rotate-half pairing, absolute positions)
# ---------------------------------------------------------------------------

def rope(x_bits, pos, theta) -> np.ndarray:
    """Rotate each head of x[T, nh, D] by its token's absolute position.

    For i < D/2 the pair (x_i, x_{i+D/2}) is rotated by angle pos * theta**(-2i/D).
    Positions are absolute, never chunk-relative, so a token's rotation does
    not depend on how its prompt was split into chunks ("Receipts", first
    paragraph: output independent of the prompt cache and run-ahead).
    """
    x = bf16_decode(x_bits)
    d = x.shape[-1]
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    omega = np.power(float(theta), -2.0 * i / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * omega[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    x1 = x[..., :half]
    x2 = x[..., half:]
    y = np.empty_like(x)
    y[..., :half] = x1 * c - x2 * s
    y[..., half:] = x2 * c + x1 * s
    return bf16_round(y)


# ---------------------------------------------------------------------------
# attention ("technical": attention made invariant with a fixed KV split
# size; the split only reorders an exact sum, so the oracle never splits)
# ---------------------------------------------------------------------------

def attention_weights(q, k, q_pos, scale):
    """Softmax weights P[h, t, s] (float64) for float64 q[T, Hq, D], k[L, Hkv, D].

    Query t of head h sees key s iff s <= q_pos[t]; head h reads kv head
    h // (Hq / Hkv).
    """
    t_n, hq, _ = q.shape
    l_n, hkv, _ = k.shape
    grp = hq // hkv
    pos = np.asarray(q_pos, dtype=np.int64)
    visible = np.arange(l_n)[None, :] <= pos[:, None]  # [T, L]
    out = np.empty((hq, t_n, l_n), dtype=np.float64)
    for h in range(hq):
        z = (q[:, h, :] @ k[:, h // grp, :].T) * scale
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        w = np.exp(z)
        out[h] = w / w.sum(axis=1, keepdims=True)
    return out


def attention(q_bits, k_bits, v_bits, q_pos, scale) -> np.ndarray:
    """o[t, h, :] = bf16( sum_{s <= q_pos[t]} softmax_s(q_t . k_s * scale) v_s ).

    q[T, Hq, D]; k, v[L, Hkv, D] with key s at absolute position s.
    ``scale`` is taken exactly as given (the library receives it as float32).
    """
    q = bf16_decode(q_bits)
    k = bf16_decode(k_bits)
    v = bf16_decode(v_bits)
    t_n, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    pos = np.asarray(q_pos, dtype=np.int64)
    if np.any(pos < 0) or np.any(pos >= k.shape[0]):
        raise ValueError("query position outside the key range")
    visible = np.arange(k.shape[0])[None, :] <= pos[:, None]
    o = np.empty((t_n, hq, d), dtype=np.float64)
    for h in range(hq):
        g = h // grp
        z = (q[:, h, :] @ k[:, g, :].T) * float(scale)
        z = np.where(visible, z, -np.inf)
        z = z - z.max(axis=1, keepdims=True)
        w = np.exp(z)
        o[:, h, :] = (w @ v[:, g, :]) / w.sum(axis=1, keepdims=True)
    return bf16_round(o)


def decode_attention(q_bits, k_bits, v_bits, scale) -> np.ndarray:
    """One decode query q[Hq, D] over all L cached keys k, v[L, Hkv, D]."""
    q = np.asarray(q_bits)[None]
    L = np.asarray(k_bits).shape[0]
    return attention(q, k_bits, v_bits, [L - 1], scale)[0]


# ---------------------------------------------------------------------------
# elementwise steps of the block
# ---------------------------------------------------------------------------

def residual_add(x_bits, o_bits) -> np.ndarray:
    """h = bf16(x + o)."""
    return bf16_round(bf16_decode(x_bits) + bf16_decode(o_bits))


def swiglu(g_bits, u_bits) -> np.ndarray:
    """act = bf16(silu(g) * u) with silu(g) = g / (1 + exp(-g))."""
    g = bf16_decode(g_bits)
    u = bf16_decode(u_bits)
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return bf16_round(silu * u)


# ---------------------------------------------------------------------------
# the pre-norm decoder block
# ---------------------------------------------------------------------------

def _linear(a_bits, w):
    """GEMM with a bf16 weight (bits array) or an int4 weight (a (wq, ws) tuple)."""
    if isinstance(w, tuple):
        return gemm_w4(a_bits, w[0], w[1])
    return gemm(a_bits, w)


def block_forward(cfg, weights, x_bits, seqs, k_pool, v_pool):
    """One forward step of a pre-norm decoder block over a batch of sequences.

    cfg: dict with hidden, n_q_heads, n_kv_heads, head_dim, ffn (0: no FFN),
        eps, rope_theta (0: no rotary embedding).
    weights: dict with gamma1, gamma2 (bf16 bits), w_qkv [(Hq+2Hkv)D, H],
        w_o [H, Hq D], w_gate_up [2F, H] (rows 0..F-1 gate, F..2F-1 up),
        w_down [H, F]; each weight is bf16 bits or an int4 (wq, ws) tuple.
    x_bits: [M, H] token rows, sequences concatenated in order.
    seqs: list of dicts {q_len, ctx_len, kv_base}; sequence i owns rows
        sum(q_len[:i]) .. + q_len[i] at absolute positions ctx_len ..
        ctx_len + q_len - 1, and its position p lives in pool row kv_base + p.
    k_pool, v_pool: [rows, Hkv, D] bf16 bits, updated in place with the new
        keys and values (positions < ctx_len must already be there).

    Every arrow is a bf16 rounding point:
    x -> n1 = RMSNorm(x, g1) -> qkv = n1 Wqkv^T -> (q, k) = RoPE(q, k), append
    k, v -> a = Attn(q, cache) -> o = a Wo^T -> h = x + o -> n2 = RMSNorm(h, g2)
    -> (g, u) = n2 Wgu^T -> act = silu(g) u -> d = act Wdown^T -> y = h + d.
    Without an FFN the block ends at h.  Returns a dict of every stage.
    """
    H = cfg["hidden"]
    hq, hkv, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
    F = cfg.get("ffn", 0)
    theta = cfg.get("rope_theta", 0.0)
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    M = x_bits.shape[0]
    st = {}
    st["n1"] = rmsnorm(x_bits, weights["gamma1"], cfg["eps"])
    st["qkv"] = _linear(st["n1"], weights["w_qkv"])
    qkv = st["qkv"].reshape(M, hq + 2 * hkv, d)
    q = qkv[:, :hq, :]
    k = qkv[:, hq:hq + hkv, :]
    v = qkv[:, hq + hkv:, :]
    pos = np.concatenate([np.arange(s["ctx_len"], s["ctx_len"] + s["q_len"]) for s in seqs])
    if theta:
        q = rope(q, pos, theta)
        k = rope(k, pos, theta)
    st["q"] = np.ascontiguousarray(q).reshape(M, hq * d)
    st["k"] = np.ascontiguousarray(k).reshape(M, hkv * d)
    st["v"] = np.ascontiguousarray(v).reshape(M, hkv * d)
    attn = np.empty((M, hq, d), dtype=np.uint16)
    row = 0
    scale = 1.0 / np.sqrt(d)
    for s in seqs:
        n, c, base = s["q_len"], s["ctx_len"], s["kv_base"]
        k_pool[base + c:base + c + n] = k[row:row + n]
        v_pool[base + c:base + c + n] = v[row:row + n]
        kc = k_pool[base:base + c + n]
        vc = v_pool[base:base + c + n]
        attn[row:row + n] = attention(q[row:row + n], kc, vc, np.arange(c, c + n), scale)
        row += n
    st["attn"] = attn.reshape(M, hq * d)
    st["o"] = _linear(st["attn"], weights["w_o"])
    st["h"] = residual_add(x_bits, st["o"])
    if not F:
        st["y"] = st["h"]
        return st
    st["n2"] = rmsnorm(st["h"], weights["gamma2"], cfg["eps"])
    st["gu"] = _linear(st["n2"], weights["w_gate_up"])
    st["act"] = swiglu(st["gu"][:, :F], st["gu"][:, F:])
    st["d"] = _linear(st["act"], weights["w_down"])
    st["y"] = residual_add(st["h"], st["d"])
    return st
