"""Helpers for the GPU tests (device setup, bit extraction, printing the case)."""
import sys

import numpy as np
import pytest
import torch

from invariant_deterministic_amd import bi


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU (torch.cuda.is_available() is False)")
    bi.lib()  # loud failure if the HIP library is missing
    return torch.device("cuda:0")


def announce(*parts):
    print("[case]", *parts, flush=True)
    sys.stdout.flush()


def bits(t):
    torch.cuda.synchronize()
    return bi.to_bits(t)


def dev(b):
    return bi.to_dev(b, "cuda:0")


def assert_bitwise(a, b, what=""):
    a = np.asarray(a); b = np.asarray(b)
    if a.shape != b.shape or not np.array_equal(a, b):
        diff = np.argwhere(a != b) if a.shape == b.shape else None
        first = tuple(diff[0]) if diff is not None and len(diff) else None
        n = len(diff) if diff is not None else "shape"
        raise AssertionError(f"{what}: not bitwise equal ({n} differing, first at {first})")


def nan_filled(shape, dtype, device="cuda"):
    """A device tensor whose every byte is 0xFF (NaN for bf16 and fp32): an output or
    workspace a kernel forgets to write, or reads before writing, shows up as NaN."""
    t = torch.empty(shape, dtype=dtype, device=device)
    t.view(torch.uint8).fill_(0xFF)
    return t


def forward_poisoned(blk, x, seqs, k_pool, v_pool):
    """Block.forward with a NaN-filled workspace and output (the stage views stay valid)."""
    lay = bi.block_workspace(blk.cfg, seqs)
    ws = nan_filled((max(int(lay.total), 256),), torch.uint8, x.device)
    y = nan_filled(tuple(x.shape), torch.bfloat16, x.device)
    return blk.forward(x, seqs, k_pool, v_pool, y=y, ws=ws)


def split_rows(y_bits, seqs):
    """Per-sequence row blocks of a block output."""
    out, row = [], 0
    for s in seqs:
        out.append(y_bits[row:row + int(s["q_len"])])
        row += int(s["q_len"])
    return out
