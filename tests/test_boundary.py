"""CPU tests of the C-ABI boundary: the library loads, exports every function
include/bi.h declares, and its argument checks return the documented status
without launching anything (no GPU is touched: every call here fails its
checks before any HIP call, or is a host-only helper)."""
import ctypes
import os
import re

import numpy as np
import pytest

from invariant_deterministic_amd import bi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, SHAPE, UNSUP, ALIGN, WS = 0, 1, 2, 3, 4, 5
P16 = ctypes.c_void_p(0x100000)     # aligned fake addresses: never dereferenced
P16b = ctypes.c_void_p(0x200000)
P16c = ctypes.c_void_p(0x300000)
MIS = ctypes.c_void_p(0x100002)     # misaligned
NUL = ctypes.c_void_p(0)


def declared_functions():
    src = open(os.path.join(ROOT, "include", "bi.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(bi_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = bi.lib()
    names = declared_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(bi.exported_symbols()) == names


def test_constants_and_build_id():
    assert bi.kv_split_size() == 256
    assert bi.gemm_tile() == (256, 256, 64)
    # narrow bf16 weights get 192-wide column tiles; int4 weights and wide ones 256
    assert [bi.gemm_tile_cols(n) for n in (8, 768, 2560, 3072, 3080, 4096, 24576)] == [192] * 4 + [256] * 3
    # int4 weights: 192-wide tiles up to 4096 rows
    assert [bi.gemm_tile_cols(n, int4_weights=True) for n in (8, 2560, 4096, 4104, 6144)] == [192] * 3 + [256] * 2
    assert bi.gemm_tile_cols(0) == 0
    bid = bi.build_id()
    assert re.fullmatch(r"[0-9a-f]{16}", bid)
    for code in range(7):
        assert bi.status_str(code).startswith("BI_")


def test_rmsnorm_checks():
    L = bi.lib()
    assert L.bi_rmsnorm(NUL, P16, P16b, 4, 256, 1e-6, NUL) == NULL
    assert L.bi_rmsnorm(P16, P16b, P16c, 0, 256, 1e-6, NUL) == SHAPE
    assert L.bi_rmsnorm(P16, P16b, P16c, 4, 12, 1e-6, NUL) == UNSUP
    assert L.bi_rmsnorm(P16, P16b, P16c, 4, 16392, 1e-6, NUL) == UNSUP
    assert L.bi_rmsnorm(P16, P16b, P16c, 4, 256, -1.0, NUL) == SHAPE
    assert L.bi_rmsnorm(P16, P16b, P16c, 4, 256, float("nan"), NUL) == SHAPE
    assert L.bi_rmsnorm(MIS, P16b, P16c, 4, 256, 1e-6, NUL) == ALIGN
    assert L.bi_rmsnorm(P16, P16b, P16, 4, 256, 1e-6, NUL) == SHAPE  # in place not allowed


def test_gemm_checks():
    L = bi.lib()
    assert L.bi_gemm(NUL, P16, P16b, 1, 8, 64, NUL) == NULL
    assert L.bi_gemm(P16, P16b, P16c, 0, 8, 64, NUL) == SHAPE
    assert L.bi_gemm(P16, P16b, P16c, 1, 12, 64, NUL) == UNSUP     # N % 8
    assert L.bi_gemm(P16, P16b, P16c, 1, 8, 96, NUL) == UNSUP      # K % 64
    assert L.bi_gemm(P16, P16b, P16c, 1, 8, (1 << 22) + 64, NUL) == UNSUP  # K above 2^22
    assert L.bi_gemm(MIS, P16b, P16c, 1, 8, 64, NUL) == ALIGN
    assert L.bi_gemm_w4(P16, P16b, NUL, P16c, 1, 8, 64, NUL) == NULL
    assert L.bi_gemm_w4(P16, P16b, ctypes.c_void_p(0x400001), P16c, 1, 8, 64, NUL) == ALIGN
    assert L.bi_gemm_w4(P16, P16b, P16c, P16, 1, 8, 32, NUL) == UNSUP


def test_fused_gemm_checks():
    L = bi.lib()
    P4 = ctypes.c_void_p(0x400000)
    # residual forms: R is checked like the other operands
    assert L.bi_gemm_residual(P16, P16b, NUL, P16c, 1, 8, 64, NUL) == NULL
    assert L.bi_gemm_residual(P16, P16b, MIS, P16c, 1, 8, 64, NUL) == ALIGN
    assert L.bi_gemm_residual(P16, P16b, P4, P16c, 0, 8, 64, NUL) == SHAPE
    assert L.bi_gemm_residual(P16, P16b, P4, P16c, 1, 12, 64, NUL) == UNSUP
    assert L.bi_gemm_w4_residual(P16, P16b, NUL, P4, P16c, 1, 8, 64, NUL) == NULL
    assert L.bi_gemm_w4_residual(P16, P16b, P16c, NUL, P4, 1, 8, 64, NUL) == NULL
    assert L.bi_gemm_w4_residual(P16, P16b, ctypes.c_void_p(0x500001), P4, P16c, 1, 8, 64, NUL) == ALIGN
    assert L.bi_gemm_w4_residual(P16, P16b, P16c, MIS, P4, 1, 8, 64, NUL) == ALIGN
    # SwiGLU forms: F outputs from 2F weight rows, F a multiple of the 128-column pair tile
    assert L.bi_gemm_swiglu(NUL, P16b, P16c, 1, 128, 64, NUL) == NULL
    assert L.bi_gemm_swiglu(P16, P16b, P16c, 1, 0, 64, NUL) == SHAPE
    assert L.bi_gemm_swiglu(P16, P16b, P16c, 1, 120, 64, NUL) == UNSUP
    assert L.bi_gemm_swiglu(P16, P16b, P16c, 1, 128, 96, NUL) == UNSUP
    assert L.bi_gemm_swiglu(P16, P16b, MIS, 1, 128, 64, NUL) == ALIGN
    # bf16 gated form: (F + 128) K 2 must stay below 2^32 (32-bit operand offsets)
    assert L.bi_gemm_swiglu(P16, P16b, P16c, 1, 4096, 1 << 19, NUL) == UNSUP
    assert L.bi_gemm_w4_swiglu(P16, P16b, NUL, P16c, 1, 128, 64, NUL) == NULL
    assert L.bi_gemm_w4_swiglu(P16, P16b, P4, P16c, 1, 64, 64, NUL) == UNSUP
    assert L.bi_gemm_w4_swiglu(P16, P16b, ctypes.c_void_p(0x500001), P16c, 1, 128, 64, NUL) == ALIGN


def test_attention_checks():
    L = bi.lib()
    sc = 0.088
    assert L.bi_attn_prefill(NUL, P16, P16b, P16c, 0, 10, 32, 8, 128, sc, NUL) == NULL
    assert L.bi_attn_prefill(P16, P16, P16b, P16c, 0, 0, 32, 8, 128, sc, NUL) == SHAPE
    assert L.bi_attn_prefill(P16, P16, P16b, P16c, -1, 4, 32, 8, 128, sc, NUL) == SHAPE
    assert L.bi_attn_prefill(P16, P16, P16b, P16c, 0, 4, 32, 8, 96, sc, NUL) == UNSUP
    assert L.bi_attn_prefill(P16, P16, P16b, P16c, 0, 4, 32, 4, 128, sc, NUL) == UNSUP  # group 8
    assert L.bi_attn_prefill(P16, P16, P16b, P16c, 0, 4, 30, 8, 128, sc, NUL) == SHAPE
    assert L.bi_attn_prefill(P16, P16, P16b, P16c, 0, 4, 32, 8, 128, 0.0, NUL) == SHAPE
    assert L.bi_attn_prefill(MIS, P16, P16b, P16c, 0, 4, 32, 8, 128, sc, NUL) == ALIGN
    need = L.bi_attn_decode_workspace(4, 1000, 32, 128)
    # one fp32 record (o[D], m, l) per (request, head, run of 8 units of 256 keys)
    assert need >= 4 * 32 * 1 * 130 * 4
    assert L.bi_attn_decode_workspace(4, 4097, 32, 128) >= 4 * 32 * 3 * 130 * 4
    args = lambda ws, nbytes, B=4, maxl=1000, D=128: (P16, P16b, P16c, P16, P16b, B, maxl, 32, 8, D, sc, ws,
                                                     nbytes, P16c, NUL)
    assert L.bi_attn_decode(*args(NUL, need)) == WS
    assert L.bi_attn_decode(*args(P16, need - 1)) == WS
    assert L.bi_attn_decode(*args(P16, need, B=0)) == SHAPE
    assert L.bi_attn_decode(*args(P16, need, maxl=0)) == SHAPE
    assert L.bi_attn_decode(*args(P16, need, D=80)) == UNSUP
    assert L.bi_attn_decode(*args(P16, need, B=65535, maxl=1 << 30)) == UNSUP  # 2^24 runs at most
    assert L.bi_attn_decode(NUL, P16b, P16c, P16, P16b, 4, 1000, 32, 8, 128, sc, P16, need, P16c, NUL) == NULL


def test_elementwise_checks():
    L = bi.lib()
    assert L.bi_add(P16, P16b, P16c, 12, NUL) == UNSUP
    assert L.bi_add(P16, NUL, P16c, 16, NUL) == NULL
    assert L.bi_swiglu(P16, P16b, 4, 12, NUL) == UNSUP
    assert L.bi_rope_kv(P16, P16b, P16c, P16, P16b, P16c, 4, 32, 8, 96, 1e6, NUL) == UNSUP
    assert L.bi_rope_kv(P16, P16b, P16c, P16, P16b, P16c, 4, 32, 8, 128, -1.0, NUL) == SHAPE


SEQS = [dict(q_len=1, ctx_len=700, kv_base=0), dict(q_len=250, ctx_len=250, kv_base=1000),
        dict(q_len=1, ctx_len=0, kv_base=5000)]


def test_step_pack_layout():
    n_tok = sum(s["q_len"] for s in SEQS)
    arr = bi._seq_array(SEQS)
    nbytes = bi.lib().bi_step_meta_bytes(arr, len(SEQS))
    buf = np.zeros(nbytes, np.uint8)
    assert bi.lib().bi_step_pack(arr, len(SEQS), ctypes.c_void_p(buf.ctypes.data), nbytes - 1) == WS
    assert bi.lib().bi_step_pack(arr, len(SEQS), ctypes.c_void_p(buf.ctypes.data), nbytes) == OK
    hdr = buf[:40].view(np.int64)
    # 3 sequences, 252 tokens, 1 prefill, 2 decodes with 701 and 1 keys: 3 + 1 units, one run each
    assert list(hdr) == [3, n_tok, 1, 2, 2]
    # prefill list at 256: {q_row, kv_base, q_start, q_len}
    pf = buf[256:256 + 24]
    assert pf[:16].view(np.int64).tolist() == [1, 1000] and pf[16:24].view(np.int32).tolist() == [250, 250]
    dec_off = 256 + 256
    d0 = buf[dec_off:dec_off + 24]
    assert d0[:16].view(np.int64).tolist() == [0, 0] and d0[16:20].view(np.int32)[0] == 701
    d1 = buf[dec_off + 24:dec_off + 48]
    assert d1[:16].view(np.int64).tolist() == [251, 5000] and d1[16:20].view(np.int32)[0] == 1
    pos_off = dec_off + 256
    pos = buf[pos_off:pos_off + 4 * n_tok].view(np.int32)
    assert pos[0] == 700 and pos[1] == 250 and pos[250] == 499 and pos[251] == 0
    kv_off = pos_off + ((4 * n_tok + 255) // 256) * 256
    kvr = buf[kv_off:kv_off + 8 * n_tok].view(np.int64)
    assert kvr[0] == 700 and kvr[1] == 1250 and kvr[250] == 1499 and kvr[251] == 5000
    u_off = kv_off + ((8 * n_tok + 255) // 256) * 256
    runs = buf[u_off:u_off + 16].view(np.int32).reshape(2, 2)
    assert runs.tolist() == [[0, 0], [1, 0]]


def test_step_pack_run_list():
    """Split decode's run list: (decode request, first unit) per run of 8 units of 256 keys, the
    full runs first in request order, then the last runs by size (7 .. 1 units), each in request order."""
    seqs = [dict(q_len=1, ctx_len=5000, kv_base=0),       # 5001 keys: 20 units, runs of 8, 8, 4
            dict(q_len=7, ctx_len=0, kv_base=6000),       # a prefill
            dict(q_len=1, ctx_len=100, kv_base=7000),     # 101 keys: 1 unit
            dict(q_len=1, ctx_len=2100, kv_base=8000),    # 2101 keys: 9 units, runs of 8, 1
            dict(q_len=1, ctx_len=1791, kv_base=12000)]   # 1792 keys: 7 units
    arr = bi._seq_array(seqs)
    nbytes = bi.lib().bi_step_meta_bytes(arr, len(seqs))
    buf = np.zeros(nbytes, np.uint8)
    assert bi.lib().bi_step_pack(arr, len(seqs), ctypes.c_void_p(buf.ctypes.data), nbytes) == OK
    hdr = buf[:40].view(np.int64)
    n_tok = 11
    assert list(hdr) == [5, n_tok, 1, 4, 7]
    off = 256 + 256 + 256 + ((4 * n_tok + 255) // 256) * 256 + ((8 * n_tok + 255) // 256) * 256
    runs = buf[off:off + 7 * 8].view(np.int32).reshape(7, 2).tolist()
    # decode indices: 0 (20 units), 1 (1 unit), 2 (9 units), 3 (7 units)
    assert runs == [[0, 0], [0, 8], [2, 0], [3, 0], [0, 16], [1, 0], [2, 8]]


def test_step_pack_rejects_bad_steps():
    L = bi.lib()
    buf = np.zeros(1 << 16, np.uint8)
    for bad in ([dict(q_len=0, ctx_len=0, kv_base=0)], [dict(q_len=1, ctx_len=-1, kv_base=0)],
                [dict(q_len=1, ctx_len=0, kv_base=-5)]):
        assert L.bi_step_pack(bi._seq_array(bad), 1, ctypes.c_void_p(buf.ctypes.data), buf.size) == SHAPE
    assert L.bi_step_pack(bi._seq_array(SEQS), 0, ctypes.c_void_p(buf.ctypes.data), buf.size) == SHAPE
    assert L.bi_step_meta_bytes(bi._seq_array(SEQS), 0) == 0


def test_block_workspace_layout():
    cfg = bi.BlockConfig(2560, 32, 8, 128, 9728, 1e-6, 1e6)
    lay = bi.block_workspace(cfg, SEQS)
    M = 252
    none = ctypes.c_size_t(-1).value
    # o and d are fused into the residual sums and, with F % 128 == 0, gate/up into SwiGLU:
    # those stages are not materialised
    assert lay.o == none and lay.d == none and lay.gu == none
    offs = [lay.n1, lay.qkv, lay.q, lay.attn, lay.h, lay.n2, lay.act, lay.decode_partials]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay.qkv - lay.n1 >= M * 2560 * 2 and lay.decode_partials - lay.act >= M * 9728 * 2
    # an FFN width the paired tile cannot cover keeps the gate/up stage
    odd = bi.block_workspace(bi.BlockConfig(2560, 32, 8, 128, 9664, 1e-6, 1e6), SEQS)
    assert odd.gu != none and odd.act - odd.gu >= M * 2 * 9664 * 2
    assert lay.total >= lay.decode_partials + bi.attn_decode_workspace(2, 701, 32, 128)
    nf = bi.block_workspace(bi.BlockConfig(256, 4, 4, 64, 0), [dict(q_len=128, ctx_len=0, kv_base=0)])
    assert nf.h == ctypes.c_size_t(-1).value and nf.decode_partials == ctypes.c_size_t(-1).value


def test_block_forward_checks():
    L = bi.lib()
    cfg = bi.BlockConfig(2560, 32, 8, 128, 9728, 1e-6, 1e6).c()
    w = bi.bi_block_weights()
    w.gamma1 = P16; w.gamma2 = P16
    for f in ("qkv", "o", "gate_up", "down"):
        setattr(w, f, bi.bi_weight(0x500000, None))
    arr = bi._seq_array(SEQS)
    pool = bi.bi_kv_pool(0x600000, 0x700000, 6000)
    lay = bi.block_workspace(bi.BlockConfig(2560, 32, 8, 128, 9728, 1e-6, 1e6), SEQS)
    call = lambda cfg_=cfg, w_=w, pool_=pool, meta=P16, x=P16b, y=P16c, ws=P16, nbytes=lay.total: L.bi_block_forward(
        ctypes.byref(cfg_), ctypes.byref(w_), arr, 3, meta, ctypes.byref(pool_), x, y, ws, nbytes, NUL)
    assert call(nbytes=lay.total - 1) == WS
    assert call(meta=NUL) == NULL
    assert call(y=P16b) == SHAPE                       # y aliases x
    assert call(pool_=bi.bi_kv_pool(0x600000, 0x700000, 5000)) == SHAPE  # last sequence needs row 5000
    w2 = bi.bi_block_weights.from_buffer_copy(w); w2.down = bi.bi_weight(None, None)
    assert call(w_=w2) == NULL
    bad = bi.BlockConfig(2560, 32, 8, 96, 9728).c()
    assert call(cfg_=bad) == UNSUP
    bad = bi.BlockConfig(2560, 32, 8, 128, 9728 + 8).c()
    assert call(cfg_=bad) == UNSUP
    w4 = bi.BlockConfig(2560, 32, 8, 128, 9728, int4=True).c()
    assert call(cfg_=w4) == NULL                        # int4 weights need scales


def test_grid_limits_rejected_before_launch():
    """Sizes whose launch grid would not fit (more than 2^32 work-items along a dimension, or
    more than 65535 along y / z) return BI_ERR_UNSUPPORTED from the checks."""
    L = bi.lib()
    assert L.bi_rmsnorm(P16, P16b, P16c, (1 << 26) - 1023, 256, 1e-6, NUL) == UNSUP
    assert L.bi_rope_kv(P16, P16b, P16c, P16, P16b, P16c, 1 << 24, 32, 8, 128, 1e6, NUL) == UNSUP
    assert L.bi_kv_append_q8(P16, P16b, P16c, 1 << 26, 8, 128, P16, P16b, P16c, P16, NUL) == UNSUP
    # 2^23 query tiles of 32 positions (group 4) at the end of a long context
    assert L.bi_attn_prefill(P16, P16, P16b, P16c, 0, (1 << 28), 32, 8, 128, 0.088, NUL) == UNSUP
    assert L.bi_gemm(P16, P16b, P16c, 1 << 30, 1 << 13, 64, NUL) == UNSUP  # 2^27 tiles


def _block_call(seqs, cfg=None, rows=1 << 40):
    L = bi.lib()
    cfg = cfg or bi.BlockConfig(2560, 32, 8, 128, 9728, 1e-6, 1e6)
    w = bi.bi_block_weights()
    w.gamma1 = P16; w.gamma2 = P16
    for f in ("qkv", "o", "gate_up", "down"):
        setattr(w, f, bi.bi_weight(0x500000, None))
    arr = bi._seq_array(seqs)
    lay = bi.block_workspace(cfg, seqs)
    pool = bi.bi_kv_pool(0x600000, 0x700000, rows)
    return L.bi_block_forward(ctypes.byref(cfg.c()), ctypes.byref(w), arr, len(seqs), P16, ctypes.byref(pool), P16b,
                              P16c, P16, lay.total, NUL)


def test_block_forward_grid_limits():
    """bi_block_forward checks every launch's grid before the first kernel is enqueued:
    too many decode requests for the combine grid, too many tokens for the RoPE grid, a decode
    longer than 2^30 keys."""
    many = [dict(q_len=1, ctx_len=10, kv_base=20 * i) for i in range(65536)]
    assert _block_call(many) == UNSUP
    assert _block_call([dict(q_len=1 << 24, ctx_len=0, kv_base=0)], bi.BlockConfig(256, 4, 4, 64)) == UNSUP
    assert _block_call([dict(q_len=1, ctx_len=(1 << 30), kv_base=0)]) == UNSUP


class _Fake:
    """Stand-in for a tensor in the CPU tests of Block.check_args (shape checks come first)."""


def test_block_binding_checks_shapes_before_launch():
    """Block.forward checks x, y and the pools against the configuration before it calls the
    library (a mismatch would make the kernels read or write out of bounds)."""
    torch = pytest.importorskip("torch")
    cfg = bi.BlockConfig(256, 4, 2, 64, 0)
    blk = bi.Block(cfg, {"gamma1": torch.zeros(256, dtype=torch.bfloat16),
                         "w_qkv": torch.zeros((512, 256), dtype=torch.bfloat16),
                         "w_o": torch.zeros((256, 256), dtype=torch.bfloat16)})
    seqs = [dict(q_len=3, ctx_len=0, kv_base=0), dict(q_len=1, ctx_len=5, kv_base=16)]
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    kp = torch.zeros((32, 2, 64), dtype=torch.bfloat16)
    bad = [
        dict(x=torch.zeros((5, 256), dtype=torch.bfloat16)),            # rows != sum of q_len
        dict(x=torch.zeros((4, 128), dtype=torch.bfloat16)),            # width != hidden
        dict(y=torch.zeros((3, 256), dtype=torch.bfloat16)),            # y shape
        dict(k_pool=torch.zeros((32, 4, 32), dtype=torch.bfloat16)),    # other head layout
        dict(v_pool=torch.zeros((31, 2, 64), dtype=torch.bfloat16)),    # pools differ
        dict(k_pool=torch.zeros((20, 2, 64), dtype=torch.bfloat16),
             v_pool=torch.zeros((20, 2, 64), dtype=torch.bfloat16)),    # second sequence needs row 21
    ]
    for b in bad:
        args = dict(x=x, k_pool=kp, v_pool=kp.clone(), y=None)
        args.update(b)
        with pytest.raises(ValueError) as ei:
            blk.check_args(args["x"], seqs, args["k_pool"], args["v_pool"], args["y"])
        assert "device" not in str(ei.value), ei.value
    # right shapes on the host: rejected as not device tensors, still before any launch
    with pytest.raises(ValueError, match="device"):
        blk.forward(x, seqs, kp, kp.clone())
    with pytest.raises(TypeError):
        blk.check_args(x, seqs, kp, kp.clone(), y=_Fake())


def test_noalloc_decode_checks():
    """bi_attn_decode_noalloc refuses, before any launch, a step whose partials would not fit
    the library's 32 MiB scratch, and otherwise checks as bi_attn_decode."""
    L = bi.lib()
    args = lambda B=4, maxl=1000, D=128, q=P16: (q, P16b, P16c, P16, P16b, B, maxl, 32, 8, D, 0.088, P16c, NUL)
    assert bi.attn_decode_workspace(1024, 32768, 32, 128) > (32 << 20)
    assert L.bi_attn_decode_noalloc(*args(B=1024, maxl=32768)) == WS
    assert L.bi_attn_decode_noalloc(*args(B=0)) == SHAPE
    assert L.bi_attn_decode_noalloc(*args(D=80)) == UNSUP
    assert L.bi_attn_decode_noalloc(*args(q=NUL)) == NULL
    assert L.bi_attn_decode_noalloc(*args(q=MIS)) == ALIGN
