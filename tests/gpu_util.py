"""Helpers shared by the GPU tests: tensors from numpy values, comparison metrics."""

import math
import sys

import numpy as np

BF16_TOL = 2e-2   # relative Frobenius error of O_t vs the fp64 oracle, bf16 NS products
F32_TOL = 1e-4    # same, fp32 NS products


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype):
    """numpy float32 values -> torch cuda tensor (bf16 values must already be bf16-exact)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dtype)
    return t.cuda()


def to_np(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy()


def bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def rel_fro(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(np.asarray(got, dtype=np.float64) - ref) / (den if den > 0 else 1.0))


def assert_bitexact(got, ref, what):
    g, r = bits(got), bits(ref)
    same = (g == r) | (np.isnan(got) & np.isnan(ref))
    if not np.all(same):
        idx = np.argwhere(~same)[:5]
        detail = [(tuple(i), float(np.asarray(got)[tuple(i)]), float(np.asarray(ref)[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int((~same).sum())} mismatches, first {detail}")


def scale_of(rows, cols, gamma):
    return math.sqrt(max(rows, cols)) * gamma


def pair_hi(x):
    """The bf16 hi of the Newton-Schulz pair (hi, 8-bit residual) as the kernels
    store X: the top 16 bits of x's fp32 bit pattern plus 0x8080 (x rounded to
    the nearest bf16, low halves from 0x7f80 rounding up; the pattern capped at
    0x7fff7f7f and the sum saturated, which only NaNs reach), as float32."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
    y = np.minimum((np.minimum(b, 0x7FFF7F7F) & 0xFFFFFFFF) + 0x8080, 0xFFFFFFFF)
    return ((y >> 16) << 16).astype(np.uint32).view(np.float32)

