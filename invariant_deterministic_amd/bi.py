"""ctypes binding of libbi.so (argument marshalling only).

Every computation runs in the library's HIP kernels; this module only checks
tensor dtypes/devices, passes raw device pointers and the current HIP stream,
and turns error codes into exceptions.  PyTorch supplies device memory and
streams.  There is no fallback: if libbi.so is missing or fails to load, every
call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbi.so")

BI_WEIGHTS_BF16 = 0
BI_WEIGHTS_INT4_G32 = 1

c_void_p = ctypes.c_void_p
c_int = ctypes.c_int
c_int64 = ctypes.c_int64
c_size_t = ctypes.c_size_t
c_float = ctypes.c_float
c_double = ctypes.c_double


class BiError(RuntimeError):
    pass


class bi_block_cfg(ctypes.Structure):
    _fields_ = [("hidden", c_int), ("n_q_heads", c_int), ("n_kv_heads", c_int), ("head_dim", c_int),
                ("ffn", c_int), ("eps", c_float), ("rope_theta", c_double), ("weight_format", c_int),
                ("decode_order", c_int), ("kv_format", c_int)]


class bi_weight(ctypes.Structure):
    _fields_ = [("w", c_void_p), ("scale", c_void_p)]


class bi_block_weights(ctypes.Structure):
    _fields_ = [("gamma1", c_void_p), ("gamma2", c_void_p), ("qkv", bi_weight), ("o", bi_weight),
                ("gate_up", bi_weight), ("down", bi_weight)]


class bi_seq(ctypes.Structure):
    _fields_ = [("q_len", ctypes.c_int32), ("ctx_len", ctypes.c_int32), ("kv_base", ctypes.c_int64)]


class bi_kv_pool(ctypes.Structure):
    _fields_ = [("k", c_void_p), ("v", c_void_p), ("rows", c_int64), ("k_scale", c_void_p), ("v_scale", c_void_p),
                ("page_table", c_void_p), ("page_entries", c_int64)]


class bi_sampling(ctypes.Structure):
    _fields_ = [("temperature", c_float), ("top_k", c_int), ("top_p", c_float), ("min_p", c_float),
                ("repeat_penalty", c_float), ("presence_penalty", c_float), ("frequency_penalty", c_float)]


class bi_block_ws_layout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in ("n1", "qkv", "q", "attn", "o", "h", "n2", "gu", "act", "d", "kv_new",
                                        "decode_partials", "total")]


# name -> (restype, argtypes), mirroring include/bi.h
_SIGNATURES = {
    "bi_status_str": (ctypes.c_char_p, [c_int]),
    "bi_build_id": (ctypes.c_char_p, []),
    "bi_kv_split_size": (c_int, []),
    "bi_gemm_tile": (None, [ctypes.POINTER(c_int)]),
    "bi_gemm_tile_cols": (c_int, [c_int64, c_int]),
    "bi_rmsnorm": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_float, c_void_p]),
    "bi_gemm": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p]),
    "bi_gemm_w4": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p]),
    "bi_gemm_residual": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p]),
    "bi_gemm_swiglu": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int64, c_void_p]),
    "bi_gemm_w4_residual": (c_int, [c_void_p] * 5 + [c_int64, c_int64, c_int64, c_void_p]),
    "bi_gemm_w4_swiglu": (c_int, [c_void_p] * 4 + [c_int64, c_int64, c_int64, c_void_p]),
    "bi_add": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_void_p]),
    "bi_swiglu": (c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p]),
    "bi_rope_kv": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int,
                           c_int, c_int, c_double, c_void_p]),
    "bi_attn_prefill": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_int, c_int,
                                c_int, c_float, c_void_p]),
    "bi_attn_decode_workspace": (c_size_t, [c_int, c_int64, c_int, c_int]),
    "bi_attn_decode": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int64, c_int,
                               c_int, c_int, c_float, c_void_p, c_size_t, c_void_p, c_void_p]),
    "bi_attn_decode_noalloc": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int64, c_int,
                                       c_int, c_int, c_float, c_void_p, c_void_p]),
    "bi_attn_decode_prefill_order": (c_int, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int,
                                             c_int64, c_int, c_int, c_int, c_float, c_void_p, c_void_p]),
    "bi_kv_append_q8": (c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int, c_int, c_void_p, c_void_p, c_void_p,
                                c_void_p, c_void_p]),
    "bi_attn_prefill_paged_q8": (c_int, [c_void_p] * 7 + [c_int64, c_int64, c_int, c_int, c_int, c_float, c_void_p]),
    "bi_attn_decode_paged_q8": (c_int, [c_void_p] * 6 + [c_int, c_void_p, c_void_p, c_int, c_int64, c_int, c_int,
                                                          c_int, c_float, c_void_p, c_void_p]),
    "bi_sample": (c_int, [c_void_p, c_int64, c_int64, ctypes.POINTER(bi_sampling), c_void_p, c_void_p, c_void_p,
                          c_int, c_void_p, c_void_p]),
    "bi_token_hash": (c_int, [c_void_p, c_void_p, c_void_p, c_int, c_void_p, c_void_p]),
    "bi_step_meta_bytes": (c_size_t, [ctypes.POINTER(bi_seq), c_int]),
    "bi_step_pack": (c_int, [ctypes.POINTER(bi_seq), c_int, c_void_p, c_size_t]),
    "bi_block_workspace": (c_int, [ctypes.POINTER(bi_block_cfg), ctypes.POINTER(bi_seq), c_int,
                                   ctypes.POINTER(bi_block_ws_layout)]),
    "bi_block_forward": (c_int, [ctypes.POINTER(bi_block_cfg), ctypes.POINTER(bi_block_weights),
                                 ctypes.POINTER(bi_seq), c_int, c_void_p, ctypes.POINTER(bi_kv_pool),
                                 c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
}

_lib = None


def lib():
    """Load libbi.so once (raises if it is missing: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise BiError(f"{LIB_PATH} is not built; run `python -m invariant_deterministic_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


def status_str(code: int) -> str:
    return lib().bi_status_str(code).decode()


def _check(code: int, what: str):
    if code != 0:
        raise BiError(f"{what}: {status_str(code)}")


def build_id() -> str:
    return lib().bi_build_id().decode()


def kv_split_size() -> int:
    return lib().bi_kv_split_size()


def gemm_tile():
    arr = (c_int * 3)()
    lib().bi_gemm_tile(arr)
    return tuple(arr)


def gemm_tile_cols(N: int, int4_weights: bool = False) -> int:
    """Column-tile width the GEMMs use for a weight of N rows (a function of N alone)."""
    return int(lib().bi_gemm_tile_cols(int(N), 1 if int4_weights else 0))


def _stream():
    return c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return c_void_p(t.data_ptr()) if t is not None else c_void_p(0)


def _dev(t: torch.Tensor, dtype, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return t


def _out(out, shape, dtype, like, name="out"):
    """A new output tensor, or the caller's after checking it: same device kind, dtype,
    contiguity and exact shape (the kernels write exactly that many elements)."""
    shape = tuple(int(v) for v in shape)
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    _dev(out, dtype, name)
    if tuple(out.shape) != shape:
        raise ValueError(f"{name}: shape {tuple(out.shape)}, expected {shape}")
    return out


BF16 = torch.bfloat16
HALF_BITS = (torch.float16, torch.int16)


# ----------------------------------------------------------------- kernels
def rmsnorm(x, gamma, eps: float, out=None):
    _dev(x, BF16, "x"); _dev(gamma, BF16, "gamma")
    rows, hidden = x.shape
    out = _out(out, x.shape, BF16, x)
    _check(lib().bi_rmsnorm(_ptr(x), _ptr(gamma), _ptr(out), rows, hidden, eps, _stream()), "bi_rmsnorm")
    return out


def gemm(A, W, out=None):
    _dev(A, BF16, "A"); _dev(W, BF16, "W")
    M, K = A.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("K mismatch")
    out = _out(out, (M, N), BF16, A)
    _check(lib().bi_gemm(_ptr(A), _ptr(W), _ptr(out), M, N, K, _stream()), "bi_gemm")
    return out


def gemm_w4(A, Wq, Ws, out=None):
    _dev(A, BF16, "A"); _dev(Wq, torch.uint8, "Wq"); _dev(Ws, HALF_BITS, "Ws")
    M, K = A.shape
    N = Wq.shape[0]
    if Wq.shape[1] * 2 != K or Ws.shape != (N, K // 32):
        raise ValueError("int4 weight shape mismatch")
    out = _out(out, (M, N), BF16, A)
    _check(lib().bi_gemm_w4(_ptr(A), _ptr(Wq), _ptr(Ws), _ptr(out), M, N, K, _stream()), "bi_gemm_w4")
    return out


def gemm_residual(A, W, R, out=None):
    """out = R + A W^T (bf16), the residual add fused into the GEMM's epilogue."""
    _dev(A, BF16, "A"); _dev(W, BF16, "W"); _dev(R, BF16, "R")
    M, K = A.shape
    N = W.shape[0]
    if W.shape[1] != K or R.shape != (M, N):
        raise ValueError("shape mismatch")
    out = _out(out, (M, N), BF16, A)
    _check(lib().bi_gemm_residual(_ptr(A), _ptr(W), _ptr(R), _ptr(out), M, N, K, _stream()), "bi_gemm_residual")
    return out


def gemm_swiglu(A, W, out=None):
    """act = swiglu(A W_gate^T, A W_up^T) for W [2F, K] (gate rows, then up rows)."""
    _dev(A, BF16, "A"); _dev(W, BF16, "W")
    M, K = A.shape
    F = W.shape[0] // 2
    if W.shape[1] != K or W.shape[0] != 2 * F:
        raise ValueError("shape mismatch")
    out = _out(out, (M, F), BF16, A)
    _check(lib().bi_gemm_swiglu(_ptr(A), _ptr(W), _ptr(out), M, F, K, _stream()), "bi_gemm_swiglu")
    return out


def gemm_w4_residual(A, Wq, Ws, R, out=None):
    _dev(A, BF16, "A"); _dev(Wq, torch.uint8, "Wq"); _dev(Ws, HALF_BITS, "Ws"); _dev(R, BF16, "R")
    M, K = A.shape
    N = Wq.shape[0]
    if Wq.shape[1] * 2 != K or Ws.shape != (N, K // 32) or R.shape != (M, N):
        raise ValueError("shape mismatch")
    out = _out(out, (M, N), BF16, A)
    _check(lib().bi_gemm_w4_residual(_ptr(A), _ptr(Wq), _ptr(Ws), _ptr(R), _ptr(out), M, N, K, _stream()),
           "bi_gemm_w4_residual")
    return out


def gemm_w4_swiglu(A, Wq, Ws, out=None):
    _dev(A, BF16, "A"); _dev(Wq, torch.uint8, "Wq"); _dev(Ws, HALF_BITS, "Ws")
    M, K = A.shape
    F = Wq.shape[0] // 2
    if Wq.shape[1] * 2 != K or Ws.shape != (2 * F, K // 32) or Wq.shape[0] != 2 * F:
        raise ValueError("shape mismatch")
    out = _out(out, (M, F), BF16, A)
    _check(lib().bi_gemm_w4_swiglu(_ptr(A), _ptr(Wq), _ptr(Ws), _ptr(out), M, F, K, _stream()), "bi_gemm_w4_swiglu")
    return out


def add(x, o, out=None):
    _dev(x, BF16, "x"); _dev(o, BF16, "o")
    if o.shape != x.shape:
        raise ValueError("x and o shapes differ")
    out = _out(out, x.shape, BF16, x)
    _check(lib().bi_add(_ptr(x), _ptr(o), _ptr(out), x.numel(), _stream()), "bi_add")
    return out


def swiglu(gu, out=None):
    _dev(gu, BF16, "gu")
    rows, two_f = gu.shape
    F = two_f // 2
    out = _out(out, (rows, F), BF16, gu)
    _check(lib().bi_swiglu(_ptr(gu), _ptr(out), rows, F, _stream()), "bi_swiglu")
    return out


def rope_kv(qkv, pos, kv_row, k_pool, v_pool, Hq, Hkv, D, theta, q_out=None):
    _dev(qkv, BF16, "qkv"); _dev(pos, torch.int32, "pos"); _dev(kv_row, torch.int64, "kv_row")
    _dev(k_pool, BF16, "k_pool"); _dev(v_pool, BF16, "v_pool")
    rows = qkv.shape[0]
    if qkv.dim() != 2 or qkv.shape[1] != (Hq + 2 * Hkv) * D or pos.shape != (rows,) or kv_row.shape != (rows,):
        raise ValueError("qkv / pos / kv_row shapes do not match rows, Hq, Hkv, D")
    q_out = _out(q_out, (rows, Hq * D), BF16, qkv, "q_out")
    _check(lib().bi_rope_kv(_ptr(qkv), _ptr(pos), _ptr(kv_row), _ptr(q_out), _ptr(k_pool), _ptr(v_pool),
                            rows, Hq, Hkv, D, float(theta), _stream()), "bi_rope_kv")
    return q_out


def attn_prefill(q, k_cache, v_cache, q_start, Hq, Hkv, D, scale, out=None):
    _dev(q, BF16, "q"); _dev(k_cache, BF16, "k_cache"); _dev(v_cache, BF16, "v_cache")
    T = q.shape[0]
    if k_cache.shape[0] < q_start + T:
        raise ValueError("cache shorter than q_start + T")
    out = _out(out, q.shape, BF16, q)
    _check(lib().bi_attn_prefill(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), int(q_start), T,
                                 Hq, Hkv, D, float(scale), _stream()), "bi_attn_prefill")
    return out


def attn_decode_workspace(B, max_kv_len, Hq, D) -> int:
    return int(lib().bi_attn_decode_workspace(B, max_kv_len, Hq, D))


def attn_decode(q, k_all, v_all, kv_offset, kv_len, max_kv_len, Hq, Hkv, D, scale, ws=None, out=None):
    _dev(q, BF16, "q"); _dev(k_all, BF16, "k_all"); _dev(v_all, BF16, "v_all")
    _dev(kv_offset, torch.int64, "kv_offset"); _dev(kv_len, torch.int32, "kv_len")
    B = q.shape[0]
    need = attn_decode_workspace(B, max_kv_len, Hq, D)
    if ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    out = _out(out, q.shape, BF16, q)
    _check(lib().bi_attn_decode(_ptr(q), _ptr(k_all), _ptr(v_all), _ptr(kv_offset), _ptr(kv_len), B,
                                int(max_kv_len), Hq, Hkv, D, float(scale), _ptr(ws), ws.numel(), _ptr(out),
                                _stream()), "bi_attn_decode")
    return out


def attn_decode_noalloc(q, k_all, v_all, kv_offset, kv_len, max_kv_len, Hq, Hkv, D, scale, out):
    """bi_attn_decode with the library's fixed per-device scratch as workspace; `out` must be
    given (the call allocates nothing, and neither does this wrapper)."""
    _dev(q, BF16, "q"); _dev(k_all, BF16, "k_all"); _dev(v_all, BF16, "v_all")
    _dev(kv_offset, torch.int64, "kv_offset"); _dev(kv_len, torch.int32, "kv_len")
    B = q.shape[0]
    if kv_offset.shape != (B,) or kv_len.shape != (B,):
        raise ValueError("kv_offset / kv_len must have one entry per query row")
    out = _out(out, q.shape, BF16, q)
    _check(lib().bi_attn_decode_noalloc(_ptr(q), _ptr(k_all), _ptr(v_all), _ptr(kv_offset), _ptr(kv_len), B,
                                        int(max_kv_len), Hq, Hkv, D, float(scale), _ptr(out), _stream()),
           "bi_attn_decode_noalloc")
    return out


def attn_decode_prefill_order(q, k_all, v_all, kv_offset, kv_len, max_kv_len, Hq, Hkv, D, scale,
                              order=None, out=None):
    _dev(q, BF16, "q"); _dev(k_all, BF16, "k_all"); _dev(v_all, BF16, "v_all")
    _dev(kv_offset, torch.int64, "kv_offset"); _dev(kv_len, torch.int32, "kv_len")
    if order is not None:
        _dev(order, torch.int32, "order")
    B = q.shape[0]
    out = _out(out, q.shape, BF16, q)
    _check(lib().bi_attn_decode_prefill_order(_ptr(q), _ptr(k_all), _ptr(v_all), _ptr(kv_offset), _ptr(kv_len),
                                              _ptr(order), B, int(max_kv_len), Hq, Hkv, D, float(scale),
                                              _ptr(out), _stream()), "bi_attn_decode_prefill_order")
    return out


class KvPoolQ8:
    """An int8 paged KV pool: codes [rows, Hkv, D] and float32 scales [rows, Hkv] for K and V.
    For the block, ``page_table`` (device int32) lists page indices; a sequence's bi_seq
    kv_base is the index of its first entry there."""

    PAGE = 64

    def __init__(self, pages, Hkv, D, device="cuda", page_table=None):
        rows = pages * self.PAGE
        self.pages, self.Hkv, self.D = pages, Hkv, D
        self.k = torch.zeros((rows, Hkv, D), dtype=torch.int8, device=device)
        self.v = torch.zeros_like(self.k)
        self.ks = torch.zeros((rows, Hkv), dtype=torch.float32, device=device)
        self.vs = torch.zeros_like(self.ks)
        self.page_table = page_table


def kv_append_q8(pool, k, v, dst_row):
    """Quantise bf16 rows k, v [rows, Hkv, D] into pool rows dst_row (int64 device)."""
    _dev(k, BF16, "k"); _dev(v, BF16, "v"); _dev(dst_row, torch.int64, "dst_row")
    _check(lib().bi_kv_append_q8(_ptr(k), _ptr(v), _ptr(dst_row), k.shape[0], pool.Hkv, pool.D, _ptr(pool.k),
                                 _ptr(pool.v), _ptr(pool.ks), _ptr(pool.vs), _stream()), "bi_kv_append_q8")


def attn_prefill_paged_q8(q, pool, block_table, q_start, Hq, scale, out=None):
    _dev(q, BF16, "q"); _dev(block_table, torch.int32, "block_table")
    T = q.shape[0]
    out = _out(out, q.shape, BF16, q)
    _check(lib().bi_attn_prefill_paged_q8(_ptr(q), _ptr(pool.k), _ptr(pool.v), _ptr(pool.ks), _ptr(pool.vs),
                                          _ptr(block_table), _ptr(out), int(q_start), T, Hq, pool.Hkv, pool.D,
                                          float(scale), _stream()), "bi_attn_prefill_paged_q8")
    return out


def attn_decode_paged_q8(q, pool, block_tables, kv_len, max_kv_len, Hq, scale, order=None, out=None):
    _dev(q, BF16, "q"); _dev(block_tables, torch.int32, "block_tables"); _dev(kv_len, torch.int32, "kv_len")
    if order is not None:
        _dev(order, torch.int32, "order")
    B = q.shape[0]
    out = _out(out, q.shape, BF16, q)
    _check(lib().bi_attn_decode_paged_q8(_ptr(q), _ptr(pool.k), _ptr(pool.v), _ptr(pool.ks), _ptr(pool.vs),
                                         _ptr(block_tables), block_tables.shape[1], _ptr(kv_len), _ptr(order), B,
                                         int(max_kv_len), Hq, pool.Hkv, pool.D, float(scale), _ptr(out), _stream()),
           "bi_attn_decode_paged_q8")
    return out


def sample(logits, seeds, positions, temperature=0.0, top_k=1, top_p=1.0, min_p=0.0, repeat=1.0,
           presence=0.0, frequency=0.0, history=None, out=None):
    """Next token per row of bf16 logits [rows, vocab]; seeds uint64-as-int64 and positions int64 [rows]."""
    _dev(logits, BF16, "logits"); _dev(seeds, torch.int64, "seeds"); _dev(positions, torch.int64, "positions")
    rows, vocab = logits.shape
    n_hist = 0
    if history is not None:
        _dev(history, torch.int32, "history")
        n_hist = history.shape[1]
    out = _out(out, (rows,), torch.int32, logits)
    prm = bi_sampling(temperature, top_k, top_p, min_p, repeat, presence, frequency)
    _check(lib().bi_sample(_ptr(logits), rows, vocab, ctypes.byref(prm), _ptr(seeds), _ptr(positions), _ptr(history),
                           n_hist, _ptr(out), _stream()), "bi_sample")
    return out


def token_hash(ids, offsets, counts, out=None):
    """BLAKE3 of each sequence's int32 ids (device); returns uint8 [n_seqs, 32]."""
    _dev(ids, torch.int32, "ids"); _dev(offsets, torch.int64, "offsets"); _dev(counts, torch.int32, "counts")
    n = counts.shape[0]
    out = _out(out, (n, 32), torch.uint8, ids)
    _check(lib().bi_token_hash(_ptr(ids), _ptr(offsets), _ptr(counts), n, _ptr(out), _stream()), "bi_token_hash")
    return out


# ------------------------------------------------------------------ block
@dataclass
class BlockConfig:
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int = 0
    eps: float = 1e-6
    rope_theta: float = 0.0
    int4: bool = False
    decode_prefill_order: bool = False  # decode in the prefill kernel's key order
    kv_q8: bool = False                 # paged int8 KV cache (needs decode_prefill_order)

    def c(self):
        return bi_block_cfg(self.hidden, self.n_q_heads, self.n_kv_heads, self.head_dim, self.ffn,
                            self.eps, float(self.rope_theta),
                            BI_WEIGHTS_INT4_G32 if self.int4 else BI_WEIGHTS_BF16,
                            1 if self.decode_prefill_order else 0, 1 if self.kv_q8 else 0)


def _seq_array(seqs):
    arr = (bi_seq * len(seqs))()
    for i, s in enumerate(seqs):
        arr[i] = bi_seq(int(s["q_len"]), int(s["ctx_len"]), int(s["kv_base"]))
    return arr


def step_meta(seqs, device="cuda"):
    """Pack a step description on the host and upload it (a device uint8 tensor)."""
    arr = _seq_array(seqs)
    nbytes = lib().bi_step_meta_bytes(arr, len(seqs))
    if nbytes == 0:
        raise BiError("bi_step_meta_bytes: invalid step")
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=torch.cuda.is_available())
    _check(lib().bi_step_pack(arr, len(seqs), c_void_p(host.data_ptr()), nbytes), "bi_step_pack")
    return host.to(device, non_blocking=True), arr


def block_workspace(cfg: BlockConfig, seqs):
    arr = _seq_array(seqs)
    lay = bi_block_ws_layout()
    c = cfg.c()
    _check(lib().bi_block_workspace(ctypes.byref(c), arr, len(seqs), ctypes.byref(lay)), "bi_block_workspace")
    return lay


class Block:
    """A decoder block whose weights live in device tensors.

    weights: dict with gamma1, gamma2 (bf16 [H]); w_qkv, w_o, w_gate_up, w_down as
    bf16 [N, K] tensors, or (for int4) (uint8 [N, K/2], fp16-bits [N, K/32]) tuples.
    """

    def __init__(self, cfg: BlockConfig, weights: dict):
        self.cfg = cfg
        self.weights = weights
        self._c = cfg.c()
        w = bi_block_weights()
        w.gamma1 = _ptr(weights["gamma1"])
        w.gamma2 = _ptr(weights.get("gamma2"))
        for field, key in (("qkv", "w_qkv"), ("o", "w_o"), ("gate_up", "w_gate_up"), ("down", "w_down")):
            val = weights.get(key)
            if val is None:
                continue
            if cfg.int4:
                setattr(w, field, bi_weight(val[0].data_ptr(), val[1].data_ptr()))
            else:
                setattr(w, field, bi_weight(val.data_ptr(), None))
        self._w = w

    def check_args(self, x, seqs, k_pool, v_pool, y=None, ws=None, meta=None):
        """Shape, dtype and device checks of forward()'s tensors, all before any launch: the
        library sees raw pointers only, so a short x or a pool of another head layout would
        otherwise be read and written out of bounds on the device."""
        c = self.cfg
        if not seqs:
            raise ValueError("seqs: at least one sequence")
        M = sum(int(s["q_len"]) for s in seqs)
        pools = () if c.kv_q8 else (("k_pool", k_pool), ("v_pool", v_pool))
        for name, t in (("x", x), *pools, ("y", y), ("ws", ws), ("meta", meta)):
            if t is not None and not isinstance(t, torch.Tensor):
                raise TypeError(f"{name}: expected a torch.Tensor")
        if tuple(x.shape) != (M, c.hidden):
            raise ValueError(f"x: shape {tuple(x.shape)}, expected (sum of q_len = {M}, hidden = {c.hidden})")
        if y is not None and tuple(y.shape) != tuple(x.shape):
            raise ValueError(f"y: shape {tuple(y.shape)}, expected {tuple(x.shape)}")
        kv = (c.n_kv_heads, c.head_dim)
        if c.kv_q8:
            # paged int8 pool (KvPoolQ8 with a page table) in k_pool; v_pool unused
            pool = k_pool
            if not isinstance(pool, KvPoolQ8) or pool.page_table is None:
                raise TypeError("k_pool: a KvPoolQ8 with a page_table for a paged int8 block")
            if (pool.Hkv, pool.D) != kv:
                raise ValueError(f"k_pool: heads {pool.Hkv} x {pool.D}, expected {kv[0]} x {kv[1]}")
            pt = pool.page_table
            if not isinstance(pt, torch.Tensor) or pt.dim() != 1:
                raise ValueError("page_table: a 1-D int32 device tensor")
            for s in seqs:
                need = (int(s["ctx_len"]) + int(s["q_len"]) + KvPoolQ8.PAGE - 1) // KvPoolQ8.PAGE
                if int(s["kv_base"]) + need > pt.shape[0]:
                    raise ValueError(f"sequence {s} needs page-table entries past {pt.shape[0]}")
            _dev(x, BF16, "x"); _dev(pool.k, torch.int8, "k codes"); _dev(pool.v, torch.int8, "v codes")
            _dev(pool.ks, torch.float32, "k scales"); _dev(pool.vs, torch.float32, "v scales")
            _dev(pt, torch.int32, "page_table")
            k_pool, v_pool = pool.k, pool.v
        else:
            for name, p in (("k_pool", k_pool), ("v_pool", v_pool)):
                if p.dim() != 3 or tuple(p.shape[1:]) != kv:
                    raise ValueError(f"{name}: shape {tuple(p.shape)}, expected (rows, {kv[0]}, {kv[1]})")
            if tuple(v_pool.shape) != tuple(k_pool.shape):
                raise ValueError("k_pool and v_pool shapes differ")
            for s in seqs:
                if int(s["kv_base"]) + int(s["ctx_len"]) + int(s["q_len"]) > k_pool.shape[0]:
                    raise ValueError(f"sequence {s} does not fit the pools' {k_pool.shape[0]} rows")
            _dev(x, BF16, "x"); _dev(k_pool, BF16, "k_pool"); _dev(v_pool, BF16, "v_pool")
        if y is not None:
            _dev(y, BF16, "y")
            if y.data_ptr() == x.data_ptr():
                raise ValueError("y may not alias x")
        if ws is not None:
            _dev(ws, torch.uint8, "ws")
        if meta is not None:
            _dev(meta, torch.uint8, "meta")
        for name, t in (("k_pool", k_pool), ("v_pool", v_pool), ("y", y), ("ws", ws), ("meta", meta)):
            if t is not None and t.device != x.device:
                raise ValueError(f"{name}: on {t.device}, x on {x.device}")
        return M

    def forward(self, x, seqs, k_pool, v_pool=None, y=None, ws=None, meta=None):
        """Run one step.  Returns (y, ws, layout); ws holds every intermediate stage.
        k_pool, v_pool: bf16 pools [rows, Hkv, D]; for a paged int8 block (cfg.kv_q8) a
        KvPoolQ8 with its page table in k_pool and v_pool None."""
        self.check_args(x, seqs, k_pool, v_pool, y, ws, meta)
        if meta is None:
            meta, arr = step_meta(seqs, x.device)
        else:
            arr = _seq_array(seqs)
            need = lib().bi_step_meta_bytes(arr, len(seqs))
            if need == 0 or meta.numel() < need:
                raise ValueError(f"meta: {meta.numel()} bytes, the step needs {need}")
        lay = block_workspace(self.cfg, seqs)
        if ws is None or ws.numel() < lay.total:
            ws = torch.empty(max(lay.total, 256), dtype=torch.uint8, device=x.device)
        y = torch.empty_like(x) if y is None else y
        if self.cfg.kv_q8:
            p = k_pool
            pool = bi_kv_pool(p.k.data_ptr(), p.v.data_ptr(), p.k.shape[0], p.ks.data_ptr(), p.vs.data_ptr(),
                              p.page_table.data_ptr(), p.page_table.shape[0])
        else:
            pool = bi_kv_pool(k_pool.data_ptr(), v_pool.data_ptr(), k_pool.shape[0], None, None, None, 0)
        _check(lib().bi_block_forward(ctypes.byref(self._c), ctypes.byref(self._w), arr, len(seqs),
                                      _ptr(meta), ctypes.byref(pool), _ptr(x), _ptr(y), _ptr(ws), ws.numel(),
                                      _stream()), "bi_block_forward")
        return y, ws, lay


def stage(ws, lay, name, rows, width):
    """View of one intermediate stage in the block workspace as bf16 [rows, width]."""
    off = getattr(lay, name)
    if off == ctypes.c_size_t(-1).value:
        raise KeyError(f"stage {name} not present")
    return ws[off:off + rows * width * 2].view(BF16).view(rows, width)


# ------------------------------------------------------ host <-> device
def to_dev(bits: np.ndarray, device="cuda"):
    """numpy uint16 bf16 bits -> device bf16 tensor."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(BF16).to(device)


def to_bits(t: torch.Tensor) -> np.ndarray:
    """device bf16 tensor -> numpy uint16 bits."""
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)
