"""Measurement probes beside the batch-invariant kernels (libbi_ceiling.so, declared in
include/bi_ceiling.h): what a plain streaming read and a plain bf16 matrix-core loop
sustain on the GPU at hand.  A benchmark reports them next to the published peaks;
they carry none of the method's arithmetic.  Argument marshalling only: both probes
run in the library's kernels, and a missing library raises."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_PATH = os.path.join(_HERE, "libbi_ceiling.so")

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m invariant_deterministic_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        vp, i64, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        h.bic_stream_read.restype = ci
        h.bic_stream_read.argtypes = [vp, i64, vp, ci, vp]
        h.bic_mfma_bf16.restype = ci
        h.bic_mfma_bf16.argtypes = [vp, ci, ci, vp, vp, vp]
        _lib = h
    return _lib


def _stream(torch):
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def stream_read(torch, x, grid: int):
    """XOR of the 32-bit words of each of `grid` equal spans of x's bytes (uint32 words as int32)."""
    out = torch.empty(grid, dtype=torch.int32, device=x.device)
    rc = lib().bic_stream_read(ctypes.c_void_p(x.data_ptr()), x.numel() * x.element_size(),
                               ctypes.c_void_p(out.data_ptr()), grid, _stream(torch))
    if rc != 0:
        raise RuntimeError(f"bic_stream_read returned {rc}")
    return out


def mfma_bf16(torch, src, grid: int, iters: int):
    """Per-lane accumulator sums (grid * 256 floats) and wave 0's (shader cycles, 100 MHz ticks)."""
    out = torch.empty(grid * 256, dtype=torch.float32, device=src.device)
    clk = torch.zeros(2, dtype=torch.int64, device=src.device)
    rc = lib().bic_mfma_bf16(ctypes.c_void_p(src.data_ptr()), grid, iters, ctypes.c_void_p(out.data_ptr()),
                             ctypes.c_void_p(clk.data_ptr()), _stream(torch))
    if rc != 0:
        raise RuntimeError(f"bic_mfma_bf16 returned {rc}")
    return out, clk


def _time_ms(torch, fn, reps: int) -> float:
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def stream_read_gbs(torch, nbytes: int = 4 << 30, grid: int = 16384, reps: int = 10) -> float:
    """Read bandwidth (GB/s, bytes read / time) of the streaming probe over an nbytes buffer."""
    x = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    t = _time_ms(torch, lambda: stream_read(torch, x, grid), reps)
    del x
    return nbytes / t / 1e6


def mfma_bf16_rate(torch, grid: int = 1024, iters: int = 20000, seed: int = 1) -> dict:
    """bf16 MFMA rate (TFLOP/s) with N(0, 1) operands, and wave 0's shader clock (GHz)."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    src = torch.randn(32768, dtype=torch.float32, device="cuda", generator=g).to(torch.bfloat16)
    holder = {}

    def run():
        holder["r"] = mfma_bf16(torch, src, grid, iters)

    t = _time_ms(torch, run, 3)
    cycles, ticks = (int(v) for v in holder["r"][1].cpu().tolist())
    flops = grid * 4 * iters * 16 * 32768
    return {"tflops": flops / t / 1e9, "clock_ghz": cycles / (ticks / 100e6) / 1e9 if ticks else None,
            "grid": grid, "iters": iters, "operands": "bf16 N(0,1)"}
