"""GPU test of bi_attn_decode_noalloc, the decode entry point that allocates nothing
(its workspace is the library's fixed per-device scratch): two calls in a row, the
second smaller, each bitwise equal to bi_attn_decode with a caller workspace on the
same inputs; sizes beyond the scratch are refused before any launch."""
import math

import numpy as np
import pytest
import torch

from invariant_deterministic_amd import bi, synth
from tests.gpu_util import announce, assert_bitwise, bits, dev, device, nan_filled

pytestmark = pytest.mark.gpu


def _inputs(seed, B, lo, hi, hq, hkv, d):
    lens = synth.uniform_ints(seed, B, lo, hi)
    total = int(lens.sum())
    k = synth.normal_bf16_device(seed + 1, (total, hkv, d))
    v = synth.normal_bf16_device(seed + 2, (total, hkv, d))
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    q = dev(synth.normal_bf16(seed + 3, (B, hq * d)))
    return q, k, v, torch.from_numpy(offs).cuda(), torch.from_numpy(lens.astype(np.int32)).cuda(), int(lens.max())


def test_noalloc_decode_matches_workspace_decode():
    device()
    hq, hkv, d = 32, 8, 128
    scale = 1.0 / math.sqrt(d)
    # the benched step's decode shape (256 requests, KV 513..8193), then a smaller one
    cases = [(9100, 256, 513, 8193, 8193), (9200, 48, 1, 3000, 3000)]
    for seed, B, lo, hi, max_len in cases:
        announce("decode noalloc B =", B, "lengths", lo, "..", hi)
        q, k, v, offs, lens, _ = _inputs(seed, B, lo, hi, hq, hkv, d)
        ref = bits(bi.attn_decode(q, k, v, offs, lens, max_len, hq, hkv, d, scale))
        out = nan_filled((B, hq * d), torch.bfloat16)
        got = bits(bi.attn_decode_noalloc(q, k, v, offs, lens, max_len, hq, hkv, d, scale, out))
        assert_bitwise(got, ref, f"noalloc vs workspace decode, B={B}")
        assert np.isfinite(bi_vals(got)).all()
    # a workspace beyond the 32 MiB scratch is refused before anything is launched
    need = bi.attn_decode_workspace(1024, 32768, hq, d)
    assert need > (32 << 20)
    q = torch.zeros((1024, hq * d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(bi.BiError, match="WORKSPACE"):
        bi.attn_decode_noalloc(q, k, v, torch.zeros(1024, dtype=torch.int64, device="cuda"),
                               torch.ones(1024, dtype=torch.int32, device="cuda"), 32768, hq, hkv, d, scale, q.clone())


def bi_vals(b):
    return (np.asarray(b, np.uint32) << 16).view(np.float32)
