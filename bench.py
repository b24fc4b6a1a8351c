#!/usr/bin/env python3
"""Bench of the batch-invariant forward path on one MI355X.

Default (the one JSON line the driver reads): the int4-weight decoder block
(hidden 4096, 32/8 heads of 128, RoPE 1e6, SwiGLU 12288, symmetric int4 group
32 with fp16 scales) on a mixed step of 256 decode requests with cached
lengths drawn uniformly from 512..8192 plus one 2048-token prefill chunk.
A step is one bi_block_forward call: RMSNorm, int4 GEMMs, RoPE + KV append,
prefill attention, split-256 decode attention + combine, residual, SwiGLU.
Inputs are seeded and synthetic and already resident in HBM when timing
starts.  The decode attention streams ~4.6 GB of KV per step, far more than
the 256 MB Infinity Cache, so weights are not served from it across steps.

`--config` selects other workloads for profiling (they print their own line):
dense (hidden 2560 block, 4000 tokens), gemm (K = N = 4096), decode (B = 64,
L ~ U{1..32768}), norm (65536 x 4096), tiny (hidden 256 block, B = 8), copy
(a plain 1 GiB copy, the reference for scaling HBM byte counters).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # flop/s, dense bf16 MFMA


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="mixed",
                   choices=["mixed", "dense", "gemm", "decode", "norm", "tiny", "copy", "lmhead", "decode_q8",
                            "ceilings"])
    p.add_argument("--batch", type=int, default=256, help="decode requests in the mixed step")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--kernel-reps", type=int, default=10)
    p.add_argument("--warm-ms", type=float, default=30.0,
                   help="warm-up before each standalone kernel timing (0: none, a fixed launch count for profiling)")
    p.add_argument("--decode-order", default="split", choices=["split", "prefill"],
                   help="decode attention: fixed 256-key split (default) or the prefill kernel's key order")
    return p.parse_args()


# --------------------------------------------------------------- helpers
WARM_MS = 30.0


def event_time_ms(torch, fn, reps, warm_ms=None, groups=3):
    """Average duration of fn() (kernels on torch's current stream) with HIP events: after
    at least warm_ms of back-to-back warm-up calls (the clock needs a few milliseconds of
    load to reach its working frequency after the host has left the GPU idle), `groups`
    groups of `reps` back-to-back calls are timed; the median group's average is returned."""
    warm_ms = WARM_MS if warm_ms is None else warm_ms
    s = torch.cuda.current_stream()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(s)
    fn()
    end.record(s)
    end.synchronize()
    first = max(start.elapsed_time(end), 1e-3)
    for _ in range(min(2000, int(math.ceil(warm_ms / first))) if warm_ms > 0 else 0):
        fn()
    avg = []
    for _ in range(groups):
        start.record(s)
        for _ in range(reps):
            fn()
        end.record(s)
        end.synchronize()
        avg.append(start.elapsed_time(end) / reps)
    return sorted(avg)[groups // 2]


def time_steps(torch, step, steps, warmup):
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps * 1e3


def step_event_stats(torch, step, n):
    """Per-step HIP-event durations of n more steps (after the contract's timed region):
    median, min and max in ms, each step bracketed by its own pair of events."""
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(s)
        step()
        b.record(s)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in ev)
    return {"median": ts[n // 2] if n % 2 else 0.5 * (ts[n // 2 - 1] + ts[n // 2]), "min": ts[0], "max": ts[-1],
            "n": n}


def copy_ceiling_gbs(torch):
    """HBM rate of torch's plain 1 GiB device-to-device copy (bytes read + written / time):
    what a generic streaming kernel reaches on this device, beside the 8 TB/s peak."""
    n = 1 << 29
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t = event_time_ms(torch, lambda: dst.copy_(src), 10)
    del src, dst
    return 2.0 * n * 2 / t / 1e6


def measured_ceilings(torch):
    """What plain kernels sustain on this device, next to the published peaks: a streaming
    read of 4 GiB (16-byte non-temporal loads, 16 per thread in flight, 16384 work-groups; far larger
    than the 256 MB Infinity Cache) and a bf16 MFMA loop with N(0, 1)
    operands (1024 work-groups x 4 waves, 16 independent accumulators per wave), with the
    shader clock its wave 0 counted (libbi_ceiling.so)."""
    from invariant_deterministic_amd import ceiling
    rate = ceiling.mfma_bf16_rate(torch)
    return {"stream_read_gbs": ceiling.stream_read_gbs(torch), "mfma_bf16_tflops": rate["tflops"],
            "mfma_clock_ghz": rate["clock_ghz"],
            "probes": "streaming read of 4 GiB; v_mfma_f32_32x32x16_bf16 loop, bf16 N(0,1) operands"}


def cpu_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        return cpu_cores()


def recorded_traffic(roof):
    """HBM bytes per launch of the dominant kernel from the committed rocprofv3
    FETCH_SIZE / WRITE_SIZE passes (scaled by the plain-copy calibration), or None
    when that record is for another kernel or the kernel's sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "decode_split_mixed_step_traffic.json")
    if roof["bound"] != "hbm" or not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in rec["source_files"]:
        with open(os.path.join(ROOT, "invariant_deterministic_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if h.hexdigest()[:16] != rec["source_sha"]:
        return None
    return rec["traffic_bytes_per_launch"]


# ------------------------------------------------------------ workloads
def mixed_workload(torch, bi, synth, B, prefill_order=False):
    H, F, hq, hkv, d = 4096, 12288, 32, 8, 128
    w = dict(gamma1=synth.ones_bf16(H), gamma2=synth.ones_bf16(H),
             w_qkv=synth.quantize_int4_g32(504, (hq + 2 * hkv) * d, H),
             w_o=synth.quantize_int4_g32(505, H, hq * d),
             w_gate_up=synth.quantize_int4_g32(506, 2 * F, H),
             w_down=synth.quantize_int4_g32(508, H, F))
    wd = {k: bi.to_dev(v) if not isinstance(v, tuple) else
          (torch.from_numpy(v[0]).cuda(), torch.from_numpy(v[1].view("int16")).cuda()) for k, v in w.items()}
    cfg = bi.BlockConfig(H, hq, hkv, d, F, 1e-6, 1e6, int4=True, decode_prefill_order=prefill_order)
    blk = bi.Block(cfg, wd)
    lens = synth.uniform_ints(501, B, 512, 8192)
    cap = 8192 + 1
    rows = B * cap + 2048
    kp = synth.normal_bf16_device(509, (rows, hkv, d))
    vp = synth.normal_bf16_device(510, (rows, hkv, d))
    seqs = [dict(q_len=1, ctx_len=int(lens[b]), kv_base=b * cap) for b in range(B)]
    seqs.append(dict(q_len=2048, ctx_len=0, kv_base=B * cap))
    x = bi.to_dev(__import__("numpy").concatenate([synth.normal_bf16(502, (B, H)),
                                                   synth.normal_bf16(503, (2048, H))]))
    return dict(cfg=cfg, w_host=w, w_dev=wd, blk=blk, lens=lens, cap=cap, kp=kp, vp=vp, seqs=seqs, x=x,
                H=H, F=F, hq=hq, hkv=hkv, d=d, B=B)


def block_flops_bytes(H, F, hq, hkv, d, tokens, weight_bytes, prefill_T, decode_lens):
    """Algorithmic work of one block step and its roofline time: linear flops (all GEMMs),
    causal prefill-attention flops (4 D per query-key pair per head), decode K/V bytes, and
    T_roof = max(flops / MFMA peak, weight bytes / HBM) + prefill flops / MFMA peak +
    (decode bytes + x, y and KV-append bytes) / HBM, intermediate activations at zero bytes."""
    lin = 2.0 * tokens * (H * (hq + 2 * hkv) * d + hq * d * H + H * 2 * F + F * H)
    pairs = prefill_T * (prefill_T + 1) / 2.0
    att_pf = 4.0 * d * hq * pairs
    dec_bytes = sum(2.0 * (L + 1) * hkv * d * 2 for L in decode_lens)
    io_bytes = 2.0 * tokens * H * 2 + tokens * 2 * hkv * d * 2
    t_roof = (max(lin / PEAK_BF16, weight_bytes / PEAK_HBM) + att_pf / PEAK_BF16
              + dec_bytes / PEAK_HBM + io_bytes / PEAK_HBM)
    return lin, att_pf, dec_bytes, t_roof


def run_mixed(args, torch, bi, synth):
    import numpy as np
    po = args.decode_order == "prefill"
    W = mixed_workload(torch, bi, synth, args.batch, po)
    blk, x, seqs, kp, vp = W["blk"], W["x"], W["seqs"], W["kp"], W["vp"]
    meta, _ = bi.step_meta(seqs, x.device)
    lay = bi.block_workspace(W["cfg"], seqs)
    ws = torch.empty(lay.total, dtype=torch.uint8, device=x.device)
    y = torch.empty_like(x)

    def step():
        blk.forward(x, seqs, kp, vp, y=y, ws=ws, meta=meta)

    ms = time_steps(torch, step, args.steps, args.warmup)
    per_step = step_event_stats(torch, step, max(args.steps, 5))
    tokens = args.batch + 2048
    # the same step with the other decode order (same weights, cache and inputs)
    other = "split" if po else "prefill"
    blk2 = bi.Block(bi.BlockConfig(W["H"], W["hq"], W["hkv"], W["d"], W["F"], 1e-6, 1e6, int4=True,
                                   decode_prefill_order=not po), W["w_dev"])
    lay2 = bi.block_workspace(blk2.cfg, seqs)
    ws2 = torch.empty(lay2.total, dtype=torch.uint8, device=x.device)
    ms_other = time_steps(torch, lambda: blk2.forward(x, seqs, kp, vp, y=y, ws=ws2, meta=meta), args.steps,
                          args.warmup)
    H, F, hq, hkv, d = W["H"], W["F"], W["hq"], W["hkv"], W["d"]
    wbytes = sum(v[0].nbytes + v[1].nbytes for k, v in W["w_host"].items() if isinstance(v, tuple))
    lin, att_pf, dec_bytes, t_roof = block_flops_bytes(H, F, hq, hkv, d, tokens, wbytes, 2048, W["lens"])

    # ---- dominant kernels, timed alone on the step's own data and launch shape
    M = tokens
    n2 = bi.stage(ws, lay, "n2", M, H)
    wgu = W["w_dev"]["w_gate_up"]
    gu_out = torch.empty((M, 2 * F), dtype=torch.bfloat16, device=x.device)
    t_gu = event_time_ms(torch, lambda: bi.gemm_w4(n2, wgu[0], wgu[1], out=gu_out), args.kernel_reps)
    gu_flops = 2.0 * M * 2 * F * H
    q = bi.stage(ws, lay, "q", M, hq * d)[:args.batch]
    offs = torch.tensor([s["kv_base"] for s in seqs[:-1]], dtype=torch.int64, device=x.device)
    lens = torch.tensor([s["ctx_len"] + 1 for s in seqs[:-1]], dtype=torch.int32, device=x.device)
    max_len = int(max(s["ctx_len"] + 1 for s in seqs[:-1]))
    dout = torch.empty_like(q)
    if po:
        order = torch.argsort(-lens.long(), stable=True).int()
        t_dec = event_time_ms(torch, lambda: bi.attn_decode_prefill_order(
            q, kp, vp, offs, lens, max_len, hq, hkv, d, 1 / math.sqrt(d), order=order, out=dout), args.kernel_reps)
    else:
        dws = torch.empty(bi.attn_decode_workspace(args.batch, max_len, hq, d), dtype=torch.uint8, device=x.device)
        t_dec = event_time_ms(torch, lambda: bi.attn_decode(q, kp, vp, offs, lens, max_len, hq, hkv, d,
                                                            1 / math.sqrt(d), ws=dws, out=dout), args.kernel_reps)
    dec_name = "decode attention (prefill key order)" if po else "decode attention (split-256 + combine)"
    if t_dec >= t_gu:
        roof = {"kernel": dec_name, "bound": "hbm",
                "achieved": dec_bytes / (t_dec * 1e-3) / 1e9, "peak": PEAK_HBM / 1e9, "unit": "GB/s"}
    else:
        roof = {"kernel": "int4 GEMM gate/up (M=%d, N=%d, K=%d)" % (M, 2 * F, H), "bound": "mfma",
                "achieved": gu_flops / (t_gu * 1e-3) / 1e12, "peak": PEAK_BF16 / 1e12, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = recorded_traffic(roof)
    roof["kernel_ms"] = t_dec if roof["bound"] == "hbm" else t_gu
    copy_gbs = copy_ceiling_gbs(torch)
    ceil = measured_ceilings(torch)
    if roof["bound"] == "hbm":
        roof["frac_of_torch_copy"] = roof["achieved"] / copy_gbs
        roof["frac_of_stream_read"] = roof["achieved"] / ceil["stream_read_gbs"]
    else:
        roof["frac_of_mfma_sustained"] = roof["achieved"] / ceil["mfma_bf16_tflops"]

    out = {
        "metric": "batch-invariant block tokens/s",
        "value": tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "per_step_ms": per_step, "torch_copy_gbs": copy_gbs, "ceilings": ceil,
        "dtype": "bf16 activations, int4 weights, fp32 accumulation", "data": "synthetic (seeded)",
        "config": {"workload": "int4 block hidden 4096, FFN 12288, 32/8 heads x 128: mixed step of "
                               f"{args.batch} decodes (KV 512..8192) + one 2048-token prefill chunk",
                   "tokens_per_step": tokens, "decode_batch": args.batch, "prefill_chunk": 2048,
                   "decode_order": args.decode_order},
        "roofline": roof,
        "block_roofline": {"t_roof_ms": t_roof * 1e3, "frac": t_roof * 1e3 / ms,
                           "linear_gflop": lin / 1e9, "prefill_attn_gflop": att_pf / 1e9,
                           "decode_kv_gb": dec_bytes / 1e9, "weight_mb": wbytes / 1e6},
        "kernels_ms": {"gemm_w4_gate_up": t_gu, "attn_decode": t_dec},
        "variants": {f"decode_order_{other}": {"ms_per_step": ms_other, "tokens_per_s": tokens / (ms_other * 1e-3)}},
        "build_id": bi.build_id(),
    }
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline_mixed(W, bi, torch)
    return out


def cpu_baseline_mixed(W, bi, torch):
    """The oracle, as it stands, on a bounded sample of the same step: 8 decode
    requests and a 128-token prefill chunk (same weights and KV distributions)."""
    import numpy as np
    import oracle
    nd, T = 8, 128
    seqs, kp_rows, xs = [], [], []
    cap = W["cap"]
    k_np, v_np = [], []
    base = 0
    x_host = bi.to_bits(W["x"])
    for b in range(nd):
        L = int(W["lens"][b])
        kc = bi.to_bits(W["kp"][b * cap:b * cap + L])
        vc = bi.to_bits(W["vp"][b * cap:b * cap + L])
        k_np.append(np.concatenate([kc, np.zeros((1,) + kc.shape[1:], np.uint16)]))
        v_np.append(np.concatenate([vc, np.zeros((1,) + vc.shape[1:], np.uint16)]))
        seqs.append(dict(q_len=1, ctx_len=L, kv_base=base))
        base += L + 1
        xs.append(x_host[b:b + 1])
    k_np.append(np.zeros((T, W["hkv"], W["d"]), np.uint16))
    v_np.append(np.zeros((T, W["hkv"], W["d"]), np.uint16))
    seqs.append(dict(q_len=T, ctx_len=0, kv_base=base))
    xs.append(x_host[W["B"]:W["B"] + T])
    kpool, vpool = np.concatenate(k_np), np.concatenate(v_np)
    cfg = dict(hidden=W["H"], n_q_heads=W["hq"], n_kv_heads=W["hkv"], head_dim=W["d"], ffn=W["F"],
               eps=1e-6, rope_theta=1e6)
    x = np.concatenate(xs)
    t0 = time.perf_counter()
    oracle.block_forward(cfg, W["w_host"], x, seqs, kpool, vpool)
    dt = time.perf_counter() - t0
    # the sample's algorithmic flops: the block's linear layers for every token, causal prefill
    # attention, and 4 D Hq flops per cached key of each decode request
    H, F, hq, hkv, d = W["H"], W["F"], W["hq"], W["hkv"], W["d"]
    lin = 2.0 * (nd + T) * (H * (hq + 2 * hkv) * d + hq * d * H + H * 2 * F + F * H)
    att = 4.0 * d * hq * (T * (T + 1) / 2.0 + sum(float(L) + 1.0 for L in W["lens"][:nd]))
    return {"value": (nd + T) / dt, "unit": "tokens/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{nd} decode requests (KV {min(W['lens'][:nd])}..{max(W['lens'][:nd])}) + one "
                      f"{T}-token prefill chunk of the same block, fp64 numpy, {dt:.1f} s",
            "gflops_fp64": (lin + att) / dt / 1e9, "host_cores": cpu_cores(), "cpu_model": cpu_model()}


# --------------------------------------------- auxiliary workloads (profiling)
def run_gemm(args, torch, bi, synth):
    K = N = 4096
    A = synth.normal_bf16_device(201, (4096, K))
    Ws = [synth.normal_bf16_device(202 + i, (N, K)) for i in range(12)]  # rotate: 12 x 32 MB > MALL
    res = {}
    for M in (1, 7, 64, 513, 4096):
        a = A[:M].contiguous()
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        it = iter(range(10 ** 9))
        t = event_time_ms(torch, lambda: bi.gemm(a, Ws[next(it) % 12], out=c), max(args.kernel_reps, 24))
        fl = 2.0 * M * N * K
        by = 2.0 * (M * K + N * K + M * N)
        res[M] = {"ms": t, "tflops": fl / t / 1e9, "gbs": by / t / 1e6,
                  "frac": max(fl / PEAK_BF16, by / PEAK_HBM) / (t * 1e-3)}
    ceil = measured_ceilings(torch)
    for r in res.values():
        r["frac_of_mfma_sustained"] = r["tflops"] / ceil["mfma_bf16_tflops"]
    return {"metric": "bf16 GEMM K=N=4096 (no split-K, one tile)", "value": res[4096]["tflops"],
            "unit": "TFLOP/s", "config": {"workload": "C = A W^T, K = N = 4096, M in 1,7,64,513,4096"},
            "per_m": res, "ceilings": ceil, "build_id": bi.build_id()}


def run_decode(args, torch, bi, synth):
    import numpy as np
    hq, hkv, d, B = 32, 8, 128, 64
    lens = synth.uniform_ints(401, B, 1, 32768)
    total = int(lens.sum())
    k = synth.normal_bf16_device(403, (total, hkv, d))
    v = synth.normal_bf16_device(404, (total, hkv, d))
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    q = bi.to_dev(synth.normal_bf16(402, (B, hq * d)))
    od = torch.from_numpy(offs).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    out = torch.empty_like(q)
    if args.decode_order == "prefill":
        order = torch.from_numpy(np.argsort(-lens, kind="stable").astype(np.int32)).cuda()
        t = event_time_ms(torch, lambda: bi.attn_decode_prefill_order(
            q, k, v, od, ld, 32768, hq, hkv, d, 1 / math.sqrt(d), order=order, out=out), max(args.kernel_reps, 20))
    else:
        ws = torch.empty(bi.attn_decode_workspace(B, 32768, hq, d), dtype=torch.uint8, device="cuda")
        t = event_time_ms(torch, lambda: bi.attn_decode(q, k, v, od, ld, 32768, hq, hkv, d, 1 / math.sqrt(d),
                                                        ws=ws, out=out), max(args.kernel_reps, 20))
    by = float(lens.sum()) * hkv * d * 2 * 2
    return {"metric": f"decode attention GB/s ({args.decode_order})", "value": by / t / 1e6, "unit": "GB/s",
            "ms": t, "frac": by / t / 1e6 / (PEAK_HBM / 1e9),
            "config": {"workload": "B=64, L~U{1..32768}, 32/8 heads x 128"}, "build_id": bi.build_id()}


def run_norm(args, torch, bi, synth):
    """RMSNorm at 65536 x 4096 (the value), and at the blocks' own shapes: the int4 mixed
    step (2304 x 4096) and the dense block's 4000-token prefill (4000 x 2560); torch's copy
    of the same tensor (the same bytes read and written) timed beside each shape."""
    res = {}
    for M, H in ((65536, 4096), (2304, 4096), (4000, 2560)):
        x = synth.normal_bf16_device(1200 + H, (M, H))
        g = bi.to_dev(synth.normal_bf16(1201, (H,), 0.02, 1.0))
        y = torch.empty_like(x)
        t = event_time_ms(torch, lambda: bi.rmsnorm(x, g, 1e-6, out=y), max(args.kernel_reps, 20))
        tc = event_time_ms(torch, lambda: y.copy_(x), max(args.kernel_reps, 20))  # same bytes, torch's copy
        by = 2.0 * M * H * 2
        res[f"{M}x{H}"] = {"ms": t, "gbs": by / t / 1e6, "frac": by / t / 1e6 / (PEAK_HBM / 1e9),
                           "torch_copy_same_bytes_gbs": by / tc / 1e6}
        del x, y
    big = res["65536x4096"]
    return {"metric": "RMSNorm GB/s", "value": big["gbs"], "unit": "GB/s", "ms": big["ms"], "frac": big["frac"],
            "config": {"workload": "65536 x 4096 (value); 2304 x 4096 and 4000 x 2560 beside it"},
            "shapes": res, "torch_copy_gbs": copy_ceiling_gbs(torch), "build_id": bi.build_id()}


def run_dense(args, torch, bi, synth):
    import numpy as np
    H, F, hq, hkv, d = 2560, 9728, 32, 8, 128
    w = dict(gamma1=synth.ones_bf16(H), gamma2=synth.ones_bf16(H),
             w_qkv=synth.normal_bf16(302, ((hq + 2 * hkv) * d, H), 0.02),
             w_o=synth.normal_bf16(303, (H, hq * d), 0.02),
             w_gate_up=synth.normal_bf16(304, (2 * F, H), 0.02),
             w_down=synth.normal_bf16(306, (H, F), 0.02))
    blk = bi.Block(bi.BlockConfig(H, hq, hkv, d, F, 1e-6, 1e6), {k: bi.to_dev(v) for k, v in w.items()})
    x = bi.to_dev(synth.normal_bf16(301, (4000, H)))
    kp = torch.zeros((4000, hkv, d), dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    res = {}
    for chunk in (4000, 1000, 250):
        plans = []
        for s0 in range(0, 4000, chunk):
            seqs = [dict(q_len=chunk, ctx_len=s0, kv_base=0)]
            meta, _ = bi.step_meta(seqs)
            lay = bi.block_workspace(blk.cfg, seqs)
            plans.append((x[s0:s0 + chunk], seqs, meta, torch.empty(lay.total, dtype=torch.uint8, device="cuda")))

        def prefill():
            for xs, seqs, meta, ws in plans:
                blk.forward(xs, seqs, kp, vp, ws=ws, meta=meta)
        ms = time_steps(torch, prefill, args.steps, args.warmup)
        wbytes = sum(v.nbytes for k, v in w.items() if k.startswith("w_"))
        lin, att, _, t_roof = block_flops_bytes(H, F, hq, hkv, d, 4000, wbytes * (4000 // chunk), 4000, [])
        res[chunk] = {"ms": ms, "tokens_per_s": 4000 / (ms * 1e-3), "roofline_frac": t_roof * 1e3 / ms}
    return {"metric": "batch-invariant block tokens/s (dense hidden 2560, 4000-token prefill)",
            "value": res[4000]["tokens_per_s"], "unit": "tokens/s", "per_chunk": res,
            "config": {"workload": "dense bf16 block hidden 2560, FFN 9728, 32/8 x 128, 4000 tokens"},
            "build_id": bi.build_id()}


def run_tiny(args, torch, bi, synth):
    import numpy as np
    H = 256
    w = dict(gamma1=synth.ones_bf16(H), w_qkv=synth.normal_bf16(102, (768, H), 0.02),
             w_o=synth.normal_bf16(103, (H, 256), 0.02))
    blk = bi.Block(bi.BlockConfig(H, 4, 4, 64, 0), {k: bi.to_dev(v) for k, v in w.items()})
    res = {}
    for B in (1, 3, 8):
        x = bi.to_dev(synth.normal_bf16(101, (128 * B, H)))
        kp = torch.zeros((128 * B, 4, 64), dtype=torch.bfloat16, device="cuda")
        vp = torch.zeros_like(kp)
        seqs = [dict(q_len=128, ctx_len=0, kv_base=128 * i) for i in range(B)]
        meta, _ = bi.step_meta(seqs)
        lay = bi.block_workspace(blk.cfg, seqs)
        ws = torch.empty(lay.total, dtype=torch.uint8, device="cuda")
        ms = time_steps(torch, lambda: blk.forward(x, seqs, kp, vp, ws=ws, meta=meta), args.steps, args.warmup)
        res[B] = {"ms": ms, "tokens_per_s": 128 * B / (ms * 1e-3)}
    return {"metric": "tiny block tokens/s", "value": res[8]["tokens_per_s"], "unit": "tokens/s",
            "per_batch": res, "config": {"workload": "hidden 256, 4 heads x 64, T=128 per sequence"},
            "build_id": bi.build_id()}


def run_lmhead(args, torch, bi, synth):
    """The step after the block for 256 decode rows: final RMSNorm, LM head (hidden 4096,
    vocabulary 151936), seeded sampling with the receipt page's settings, token hashes."""
    import numpy as np
    B, H, V, NH = 256, 4096, 151936, 64
    x = synth.normal_bf16_device(1300, (B, H))
    g = bi.to_dev(synth.normal_bf16(1301, (H,), 0.02, 1.0))
    w = synth.normal_bf16_device(1302, (V, H), 0.02)
    rng = np.random.default_rng(1303)
    hist = torch.from_numpy(rng.integers(0, V, size=(B, NH)).astype(np.int32)).cuda()
    seeds = torch.from_numpy(rng.integers(0, 2 ** 62, size=B).astype(np.int64)).cuda()
    pos = torch.from_numpy(rng.integers(512, 8192, size=B).astype(np.int64)).cuda()
    n = torch.empty_like(x)
    logits = torch.empty((B, V), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty(B, dtype=torch.int32, device="cuda")
    seq = torch.empty((B, NH + 1), dtype=torch.int32, device="cuda")
    seq[:, :NH] = hist
    offs = torch.arange(B, dtype=torch.int64, device="cuda") * (NH + 1)
    cnts = torch.full((B,), NH + 1, dtype=torch.int32, device="cuda")
    digests = torch.empty((B, 32), dtype=torch.uint8, device="cuda")
    prm = dict(temperature=0.8, top_k=50, top_p=0.95, min_p=0.05, repeat=1.1)

    def sample():
        bi.sample(logits, seeds, pos, history=hist, out=ids, **prm)

    def step():
        bi.rmsnorm(x, g, 1e-6, out=n)
        bi.gemm(n, w, out=logits)
        sample()
        seq[:, NH] = ids
        bi.token_hash(seq, offs, cnts, out=digests)

    ms = time_steps(torch, step, args.steps, args.warmup)
    t_gemm = event_time_ms(torch, lambda: bi.gemm(n, w, out=logits), max(args.kernel_reps, 10))
    t_samp = event_time_ms(torch, sample, max(args.kernel_reps, 10))
    t_hash = event_time_ms(torch, lambda: bi.token_hash(seq, offs, cnts, out=digests), max(args.kernel_reps, 10))
    fl = 2.0 * B * V * H
    wb = 2.0 * V * H
    return {"metric": "step after the block tokens/s", "value": B / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "config": {"workload": f"final RMSNorm + LM head (hidden {H}, vocabulary {V}) + seeded sampling "
                                   f"(T 0.8, top-k 50, top-p 0.95, min-p 0.05, repeat 1.1 over {NH}) + token hashes, "
                                   f"{B} rows"},
            "kernels_ms": {"lm_head_gemm": t_gemm, "sample": t_samp, "token_hash": t_hash},
            "lm_head": {"tflops": fl / t_gemm / 1e9, "frac_mfma": fl / t_gemm / 1e9 / (PEAK_BF16 / 1e12),
                        "weight_gbs": wb / t_gemm / 1e6, "frac_hbm": wb / t_gemm / 1e6 / (PEAK_HBM / 1e9)},
            "build_id": bi.build_id()}


def run_decode_q8(args, torch, bi, synth):
    """Decode over the quantised, paged cache for the mixed step's 256 requests (KV 513..8193,
    32/8 heads x 128), in prefill key order, longest first; bf16 prefill-order decode on the same
    requests beside it."""
    import numpy as np
    hq, hkv, d, B, PG = 32, 8, 128, 256, 64
    lens = synth.uniform_ints(501, B, 512, 8192) + 1
    npg = (lens + PG - 1) // PG
    total_pages = int(npg.sum())
    rng = np.random.default_rng(1400)
    perm = rng.permutation(total_pages).astype(np.int32)
    maxp = int(npg.max())
    tables = np.zeros((B, maxp), np.int32)
    used = 0
    rows = []
    for b in range(B):
        tables[b, :npg[b]] = perm[used:used + npg[b]]
        used += int(npg[b])
        rows.append(tables[b, np.arange(lens[b]) // PG].astype(np.int64) * PG + np.arange(lens[b]) % PG)
    rows = torch.from_numpy(np.concatenate(rows)).cuda()
    pool = bi.KvPoolQ8(total_pages, hkv, d)
    n = rows.numel()
    for s0 in range(0, n, 1 << 18):        # quantise seeded bf16 keys and values into the pages
        k = synth.normal_bf16_device(1401 + s0, (min(n - s0, 1 << 18), hkv, d))
        v = synth.normal_bf16_device(1402 + s0, (min(n - s0, 1 << 18), hkv, d))
        bi.kv_append_q8(pool, k, v, rows[s0:s0 + k.shape[0]].contiguous())
    q = bi.to_dev(synth.normal_bf16(402, (B, hq * d)))
    tbl = torch.from_numpy(tables).cuda()
    ld = torch.from_numpy(lens.astype(np.int32)).cuda()
    order = torch.from_numpy(np.argsort(-lens, kind="stable").astype(np.int32)).cuda()
    out = torch.empty_like(q)
    mx = int(lens.max())
    t = event_time_ms(torch, lambda: bi.attn_decode_paged_q8(q, pool, tbl, ld, mx, hq, 1 / math.sqrt(d), order=order,
                                                             out=out), max(args.kernel_reps, 20))
    by = float(lens.sum()) * hkv * (d + 4) * 2
    # the bf16 decode in prefill order on contiguous bf16 K/V of the same lengths
    kb = synth.normal_bf16_device(403, (n, hkv, d))
    vb = synth.normal_bf16_device(404, (n, hkv, d))
    offs = torch.from_numpy(np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)).cuda()
    t16 = event_time_ms(torch, lambda: bi.attn_decode_prefill_order(q, kb, vb, offs, ld, mx, hq, hkv, d,
                                                                     1 / math.sqrt(d), order=order, out=out),
                        max(args.kernel_reps, 20))
    return {"metric": "decode attention GB/s (int8 paged cache, prefill key order)", "value": by / t / 1e6,
            "unit": "GB/s", "ms": t, "frac": by / t / 1e6 / (PEAK_HBM / 1e9),
            "bf16_same_requests": {"ms": t16, "gbs": float(lens.sum()) * hkv * d * 4 / t16 / 1e6},
            "config": {"workload": "256 requests, KV 513..8193, 32/8 heads x 128, int8 codes + fp32 scale per "
                                   "(token, head), 64-token pages in random order"}, "build_id": bi.build_id()}


def run_copy(args, torch, bi, synth):
    """A plain 1 GiB device copy (torch), the reference for scaling HBM counters."""
    n = 1 << 29
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    t = event_time_ms(torch, lambda: dst.copy_(src), 5)
    return {"metric": "plain copy GB/s", "value": 2.0 * n * 2 / t / 1e6, "unit": "GB/s", "ms": t,
            "bytes_read": n * 2, "bytes_written": n * 2, "config": {"workload": "1 GiB bf16 copy"}}


def run_ceilings(args, torch, bi, synth):
    """The two measurement probes alone (libbi_ceiling.so), for their own profiles."""
    c = measured_ceilings(torch)
    return {"metric": "measured ceilings", "value": c["stream_read_gbs"], "unit": "GB/s", **c,
            "config": {"workload": "streaming read of 4 GiB; bf16 MFMA loop, 1024 x 4 waves x 20000 rounds"}}


def main():
    global WARM_MS
    args = parse()
    WARM_MS = args.warm_ms
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch
    from invariant_deterministic_amd import bi, synth
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    bi.lib()
    fn = {"mixed": run_mixed, "dense": run_dense, "gemm": run_gemm, "decode": run_decode,
          "norm": run_norm, "tiny": run_tiny, "copy": run_copy, "lmhead": run_lmhead,
          "decode_q8": run_decode_q8, "ceilings": run_ceilings}[args.config]
    out = fn(args, torch, bi, synth)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
