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
