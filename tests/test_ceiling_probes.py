"""The measurement probes (libbi_ceiling.so, include/bi_ceiling.h) that a benchmark runs
beside the batch-invariant kernels.

CPU: the library exports exactly the functions its header declares, and its argument
checks return their documented codes without launching anything.
GPU: the streaming read's per-span XOR of 32-bit words equals the same fold computed on
the host, bit for bit (ragged spans included); the MFMA loop's per-wave sum of
accumulators equals iters times the sum of its 16 products computed in fp64 from the
operands' documented lane layout (so every MFMA the rate is counted for ran)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from invariant_deterministic_amd import ceiling

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P16 = ctypes.c_void_p(0x100000)
P16b = ctypes.c_void_p(0x200000)
P16c = ctypes.c_void_p(0x300000)
NUL = ctypes.c_void_p(0)


def test_probe_library_exports_its_header():
    src = open(os.path.join(ROOT, "include", "bi_ceiling.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    declared = sorted(set(re.findall(r"\b(bic_[a-z0-9_]+)\s*\(", src)))
    assert declared == ["bic_mfma_bf16", "bic_stream_read"]
    L = ceiling.lib()
    out = subprocess.run(["nm", "-D", "--defined-only", ceiling.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = sorted(l.split()[-1] for l in out.splitlines() if l.split()[-2:-1] == ["T"])
    assert exported == declared
    for n in declared:
        assert hasattr(L, n)


def test_probe_argument_checks():
    L = ceiling.lib()
    assert L.bic_stream_read(NUL, 1024, P16b, 4, NUL) == 1
    assert L.bic_stream_read(ctypes.c_void_p(0x100008), 1024, P16b, 4, NUL) == 1   # x not 16-byte aligned
    assert L.bic_stream_read(P16, 1024, ctypes.c_void_p(0x200002), 4, NUL) == 1    # out not 4-byte aligned
    assert L.bic_stream_read(P16, 1000, P16b, 4, NUL) == 2                         # bytes % 16
    assert L.bic_stream_read(P16, 0, P16b, 4, NUL) == 2
    assert L.bic_stream_read(P16, 1024, P16b, 0, NUL) == 2
    assert L.bic_stream_read(P16, 1024, P16b, 65537, NUL) == 2
    assert L.bic_mfma_bf16(NUL, 4, 1, P16b, P16c, NUL) == 1
    assert L.bic_mfma_bf16(P16, 4, 1, P16b, ctypes.c_void_p(0x300004), NUL) == 1   # clk not 8-byte aligned
    assert L.bic_mfma_bf16(P16, 0, 1, P16b, P16c, NUL) == 2
    assert L.bic_mfma_bf16(P16, 4, 0, P16b, P16c, NUL) == 2


def _xor_spans(words, grid):
    """Host fold: span g of grid equal spans of 16-byte words, XOR of its 32-bit words."""
    n16 = words.size // 4
    per = -(-n16 // grid)
    out = np.zeros(grid, np.uint32)
    for g in range(grid):
        lo, hi = g * per, min(g * per + per, n16)
        if lo < hi:
            out[g] = np.bitwise_xor.reduce(words[4 * lo:4 * hi])
    return out


def _mfma_wave_totals(src_bits, grid, iters):
    """fp64 sum of every accumulator of every wave: iters x sum over j of the 32 x 32 block
    product a[j % 4] x b[j / 4], with lane l holding row/column l % 32 and k = 8 (l / 32) + e."""
    frag = (src_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(4096, 8)
    totals = np.zeros(grid * 4)
    for w in range(4):
        t = 64 * w + np.arange(64)
        a = np.stack([frag[(t * 8 + i) % 4096] for i in range(4)])       # [i, lane, e]
        b = np.stack([frag[(t * 8 + 4 + i) % 4096] for i in range(4)])
        tot = 0.0
        for j in range(16):
            for h in (0, 1):
                sa = a[j % 4, 32 * h:32 * h + 32].sum(axis=0)   # sum over rows, per k = 8 h + e
                sb = b[j // 4, 32 * h:32 * h + 32].sum(axis=0)  # sum over columns, per k
                tot += float((sa * sb).sum())
        totals[w::4] = iters * tot   # every work-group runs the same operands
    return totals


@pytest.mark.gpu
def test_probes_on_gpu():
    import torch

    from tests.gpu_util import announce, device
    device()
    rng = np.random.default_rng(11)
    for nbytes, grid in ((1 << 20, 64), (1 << 20, 7), (4096 + 48, 5), (160, 64)):
        announce("stream read", nbytes, "bytes,", grid, "work-groups")
        host = rng.integers(0, 2 ** 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
        x = torch.from_numpy(host.view(np.int32)).cuda()
        got = ceiling.stream_read(torch, x, grid).cpu().numpy().view(np.uint32)
        assert np.array_equal(got, _xor_spans(host, grid))
    src = torch.from_numpy(rng.standard_normal(32768).astype(np.float32)).to(torch.bfloat16)
    src_bits = src.view(torch.int16).numpy().view(np.uint16)
    src = src.cuda()
    for grid, iters in ((2, 1), (3, 3)):
        announce("mfma probe", grid, "work-groups,", iters, "rounds")
        out, clk = ceiling.mfma_bf16(torch, src, grid, iters)
        lane = out.cpu().numpy().astype(np.float64).reshape(grid * 4, 64)
        want = _mfma_wave_totals(src_bits, grid, iters)
        scale = iters * 16 * 32 * 32 * 16 * 4.0   # bound on the sum of |products| for |x| <~ 4
        assert np.all(np.abs(lane.sum(axis=1) - want) <= 1e-6 * scale), (lane.sum(axis=1)[:4], want[:4])
        c = clk.cpu().numpy()
        assert c[0] > 0 and c[1] > 0
    rate = ceiling.mfma_bf16_rate(torch, grid=256, iters=2000)
    announce("mfma rate", rate)
    assert rate["tflops"] > 100 and 0.5 < rate["clock_ghz"] < 3.0
    gbs = ceiling.stream_read_gbs(torch, nbytes=1 << 28, reps=3)
    announce("stream read GB/s", gbs)
    assert gbs > 500
