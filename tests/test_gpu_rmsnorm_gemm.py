"""GPU parity and invariance of bi_rmsnorm, bi_gemm and bi_gemm_w4, and the fused
GEMM epilogues (residual add, SwiGLU) (through the C-ABI).

Parity: each output element within |gpu - oracle| <= 8e-3 |oracle| + 1e-3;
bitwise where the mathematics fixes the bits (constant rows, small-integer
GEMMs whose fp32 accumulation is exact in any order).  Invariance: a row's bits
are identical for every M and every position of the row in the batch.
"""
import numpy as np
import pytest
import torch

import oracle
from invariant_deterministic_amd import bi, synth
from tests.gpu_util import announce, assert_bitwise, bits, dev, device
from tests.util import assert_within_tolerance

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("rows,hidden", [(1024, 256), (4000, 2560), (2304, 4096), (37, 8), (5, 16384), (3, 520)])
def test_rmsnorm_parity(rows, hidden):
    device()
    announce("rmsnorm parity", rows, hidden)
    x = synth.normal_bf16(1000 + hidden, (rows, hidden))
    g = synth.normal_bf16(1001 + hidden, (hidden,), 0.02, 1.0)
    y = bits(bi.rmsnorm(dev(x), dev(g), 1e-6))
    assert_within_tolerance(y, oracle.rmsnorm(x, g, 1e-6), f"rmsnorm {rows}x{hidden}")


def test_rmsnorm_closed_forms():
    device()
    announce("rmsnorm closed forms")
    H = 2560
    x = np.zeros((4, H), np.uint16)
    x[0] = synth.to_bf16_bits(np.full(H, 2.0, np.float32))
    x[1] = synth.to_bf16_bits(np.full(H, -0.5, np.float32))
    x[2] = synth.to_bf16_bits(np.full(H, 3.0, np.float32))
    y = bits(bi.rmsnorm(dev(x), dev(synth.ones_bf16(H)), 1e-6))
    assert np.all(y[0] == 0x3F80) and np.all(y[1] == 0xBF80) and np.all(y[2] == 0x3F80)
    assert np.all(y[3] == 0)


def test_rmsnorm_batch_invariance():
    device()
    H = 4096
    master = synth.normal_bf16(1100, (4000, H))
    g = synth.normal_bf16(1101, (H,), 0.02, 1.0)
    gd = dev(g)
    ref = bits(bi.rmsnorm(dev(master), gd, 1e-6))
    rng = np.random.default_rng(1102)
    for M in (1, 3, 7, 64, 255, 256, 257, 1000, 4000):
        for order in ("id", "rev", "rand"):
            announce("rmsnorm invariance", M, order)
            idx = np.arange(M)
            if order == "rev":
                idx = idx[::-1].copy()
            elif order == "rand":
                idx = rng.choice(4000, size=M, replace=False)
            y = bits(bi.rmsnorm(dev(master[idx]), gd, 1e-6))
            assert_bitwise(y, ref[idx], f"rmsnorm M={M} {order}")
    # repeats
    for _ in range(10):
        assert_bitwise(bits(bi.rmsnorm(dev(master), gd, 1e-6)), ref, "rmsnorm repeat")


def test_rmsnorm_large_m_sampled():
    device()
    announce("rmsnorm M=65536 H=4096")
    M, H = 65536, 4096
    xd = synth.normal_bf16_device(1200, (M, H))
    g = synth.normal_bf16(1201, (H,), 0.02, 1.0)
    y = bi.rmsnorm(xd, dev(g), 1e-6)
    idx = np.random.default_rng(1202).choice(M, 128, replace=False)
    x_s = bits(xd[torch.from_numpy(idx).cuda()])
    y_s = bits(y[torch.from_numpy(idx).cuda()])
    assert_within_tolerance(y_s, oracle.rmsnorm(x_s, g, 1e-6), "rmsnorm 65536 sampled")
    # the sampled rows alone give the same bits
    assert_bitwise(bits(bi.rmsnorm(dev(x_s), dev(g), 1e-6)), y_s, "rmsnorm big-M rows alone")


# --------------------------------------------------------------------- GEMM
@pytest.mark.parametrize("m,n,k", [(5, 8, 64), (300, 264, 128), (513, 768, 256), (64, 4096, 4096), (1, 2560, 9728)])
def test_gemm_small_integers_bitwise(m, n, k):
    device()
    announce("gemm small-int", m, n, k)
    a = synth.small_int_bf16(2000 + m, (m, k))
    w = synth.small_int_bf16(2001 + n, (n, k))
    c = bits(bi.gemm(dev(a), dev(w)))
    assert_bitwise(c, oracle.gemm(a, w), f"gemm small-int {m}x{n}x{k}")


@pytest.mark.parametrize("m,n,k", [(257, 520, 320), (1024, 768, 256), (1024, 256, 256), (33, 6144, 2560)])
def test_gemm_parity(m, n, k):
    device()
    announce("gemm parity", m, n, k)
    a = synth.normal_bf16(2100 + m, (m, k))
    w = synth.normal_bf16(2101 + n, (n, k), 0.02 if k > 512 else 1.0)
    c = bits(bi.gemm(dev(a), dev(w)))
    assert_within_tolerance(c, oracle.gemm(a, w), f"gemm {m}x{n}x{k}")


def test_gemm_identity_weight():
    device()
    announce("gemm identity")
    a = synth.normal_bf16(2200, (300, 512))
    eye = synth.to_bf16_bits(np.eye(512, dtype=np.float32))
    assert_bitwise(bits(bi.gemm(dev(a), dev(eye))), a, "gemm A I = A")


def test_gemm_config2_invariance_and_parity():
    """K = N = 4096, M in {1, 7, 64, 513, 4096}, rows in identity / reversed / random order."""
    device()
    K = N = 4096
    A = synth.normal_bf16(201, (4096, K))
    W = synth.normal_bf16(202, (N, K))
    Wd = dev(W)
    announce("gemm config2 reference M=4096")
    ref = bits(bi.gemm(dev(A), Wd))
    rng = np.random.default_rng(203)
    for M in (1, 7, 64, 513, 4096):
        for order in ("id", "rev", "rand"):
            announce("gemm config2 invariance", M, order)
            idx = np.arange(M)
            if order == "rev":
                idx = idx[::-1].copy()
            elif order == "rand":
                idx = rng.choice(4096, size=M, replace=False)
            c = bits(bi.gemm(dev(A[idx]), Wd))
            assert_bitwise(c, ref[idx], f"gemm M={M} {order}")
    for _ in range(10):
        assert_bitwise(bits(bi.gemm(dev(A), Wd)), ref, "gemm repeat")
    # 64 sampled rows against the oracle; those rows alone at M = 1 are bitwise the same
    samp = rng.choice(4096, 64, replace=False)
    announce("gemm config2 sampled parity")
    assert_within_tolerance(ref[samp], oracle.gemm(A[samp], W), "gemm config2 sampled rows")
    for i in samp[:16]:
        assert_bitwise(bits(bi.gemm(dev(A[i:i + 1]), Wd))[0], ref[i], f"gemm row {i} alone")


# ------------------------------------------------------------------ int4 GEMM
@pytest.mark.parametrize("m,n,k", [(300, 264, 256), (70, 4096, 4096), (513, 512, 12288), (40, 4104, 256)])
def test_gemm_w4_equals_bf16_on_dequantised(m, n, k):
    device()
    announce("gemm_w4 vs bf16", m, n, k)
    a = synth.normal_bf16(3000 + m, (m, k))
    wq, ws = synth.quantize_int4_g32(3001 + n, n, k, 0.02)
    wdq = oracle.dequant_int4_g32(wq, ws)
    c4 = bits(bi.gemm_w4(dev(a), torch.from_numpy(wq).cuda(), torch.from_numpy(ws.view(np.int16)).cuda()))
    cb = bits(bi.gemm(dev(a), dev(wdq)))
    assert_bitwise(c4, cb, "int4 GEMM vs bf16 GEMM on the dequantised weight")
    assert_within_tolerance(c4, oracle.gemm_w4(a, wq, ws), f"gemm_w4 {m}x{n}x{k}")


def test_gemm_w4_small_integers_bitwise():
    device()
    announce("gemm_w4 small-int")
    n, k, m = 264, 512, 77
    rng = np.random.default_rng(3100)
    codes = rng.integers(-8, 8, size=(n, k))
    nib = (codes & 0xF).astype(np.uint8)
    wq = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    ws = np.full((n, k // 32), 0x3C00, np.uint16)
    ws[:, 1::2] = 0x4000  # scale 2 on odd groups: still exact
    a = synth.small_int_bf16(3101, (m, k))
    c = bits(bi.gemm_w4(dev(a), torch.from_numpy(wq).cuda(), torch.from_numpy(ws.view(np.int16)).cuda()))
    assert_bitwise(c, oracle.gemm_w4(a, wq, ws), "gemm_w4 small-int")


def test_gemm_w4_batch_invariance():
    device()
    K, N = 4096, 6144
    A = synth.normal_bf16(3200, (2304, K))
    wq, ws = synth.quantize_int4_g32(3201, N, K, 0.02)
    wqd, wsd = torch.from_numpy(wq).cuda(), torch.from_numpy(ws.view(np.int16)).cuda()
    ref = bits(bi.gemm_w4(dev(A), wqd, wsd))
    rng = np.random.default_rng(3202)
    # 288 / 289 / 385: a last tile row whose first 128-row wave has 32 / 33 valid rows, and one
    # whose second wave has a single valid row (the one-block and four-block paths side by side)
    for M in (1, 2, 65, 288, 289, 385, 2049, 2304):
        announce("gemm_w4 invariance", M)
        idx = rng.choice(2304, size=M, replace=False)
        assert_bitwise(bits(bi.gemm_w4(dev(A[idx]), wqd, wsd)), ref[idx], f"gemm_w4 M={M}")


# ------------------------------------------------------- fused epilogues
@pytest.mark.parametrize("m,n,k", [(1, 768, 256), (77, 2560, 1024), (300, 520, 320), (513, 4096, 4096)])
def test_gemm_residual_equals_gemm_then_add(m, n, k):
    device()
    announce("gemm + residual", m, n, k)
    a = dev(synth.normal_bf16(5000 + m, (m, k)))
    w = dev(synth.normal_bf16(5001 + n, (n, k), 0.02))
    r = dev(synth.normal_bf16(5002 + k, (m, n)))
    ref = bits(bi.add(r, bi.gemm(a, w)))
    assert_bitwise(bits(bi.gemm_residual(a, w, r)), ref, "bf16 fused residual")
    r2 = r.clone()
    bi.gemm_residual(a, w, r2, out=r2)  # in place over the residual
    assert_bitwise(bits(r2), ref, "bf16 fused residual in place")
    wq, ws = synth.quantize_int4_g32(5003 + n, n, k)
    wq, ws = torch.from_numpy(wq).cuda(), torch.from_numpy(ws.view("int16")).cuda()
    ref4 = bits(bi.add(r, bi.gemm_w4(a, wq, ws)))
    assert_bitwise(bits(bi.gemm_w4_residual(a, wq, ws, r)), ref4, "int4 fused residual")


@pytest.mark.parametrize("m,f,k", [(1, 128, 256), (77, 640, 1024), (300, 9728, 2560), (513, 12288, 4096)])
def test_gemm_swiglu_equals_gemm_then_swiglu(m, f, k):
    device()
    announce("gemm + swiglu", m, f, k)
    a = dev(synth.normal_bf16(5100 + m, (m, k)))
    w = dev(synth.normal_bf16(5101 + f, (2 * f, k), 0.02))
    ref = bits(bi.swiglu(bi.gemm(a, w)))
    got = bits(bi.gemm_swiglu(a, w))
    assert_bitwise(got, ref, "bf16 fused swiglu")
    wq, ws = synth.quantize_int4_g32(5102 + f, 2 * f, k)
    wq, ws = torch.from_numpy(wq).cuda(), torch.from_numpy(ws.view("int16")).cuda()
    ref4 = bits(bi.swiglu(bi.gemm_w4(a, wq, ws)))
    assert_bitwise(bits(bi.gemm_w4_swiglu(a, wq, ws)), ref4, "int4 fused swiglu")
    # rows of the fused form do not depend on the batch either
    if m > 1:
        one = bits(bi.gemm_w4_swiglu(a[m - 1:m], wq, ws))
        assert_bitwise(one[0], ref4[m - 1], "fused swiglu row alone")


def test_gemm_operand_above_4gib():
    """A of more than 4 GiB (2^21 + 77 rows of K = 1024): the kernel addresses operands from
    each tile's first row, so rows past the 4 GiB mark are as correct as the first ones.
    Sampled rows against the oracle, and bitwise against the same rows computed alone."""
    device()
    M, N, K = (1 << 21) + 77, 264, 1024
    announce("gemm A above 4 GiB", M, N, K)
    A = synth.normal_bf16_device(5400, (M, K))
    assert A.numel() * 2 > (1 << 32)
    w = synth.normal_bf16(5401, (N, K), 0.02)
    C = bits(bi.gemm(A, dev(w)))
    rows = np.array([0, 1, 255, 256, (1 << 20) + 3, (1 << 21) - 1, 1 << 21, M - 1])
    a_rows = bits(A[torch.from_numpy(rows).cuda()])
    del A
    assert_within_tolerance(C[rows], oracle.gemm(a_rows, w), "gemm rows past 4 GiB")
    assert_bitwise(C[rows], bits(bi.gemm(dev(a_rows), dev(w))), "rows alone")
