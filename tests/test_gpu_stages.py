"""Kernel unit tests of the three bf16 Newton-Schulz products (one step is
X <- a X + b A X + c A^2 X with A = X X^T, DeepSeek-V4 book ch. 6 section 3),
each run alone through the muon_ns_stage hook exactly as muon_step runs it for
one matrix of that shape (same tiles, same split of long K loops), and compared
element by element with fp64 products of the *same* bf16 operands:

  GRAM   A = bf16(X_hi X_hi^T)            X_hi = bf16(X)
  POLY   B = bf16(b A + c A A)            A given, rounded to bf16
  APPLY  X' = a X + B X_hi                B rounded to bf16, X kept as hi + residual

The bounds are those of the arithmetic: the final rounding to bf16 (half an
ulp of an 8-bit significand: 2^-8 relative) or to the hi + residual pair
(2^-15 relative), plus K 2^-24 times the
product of the absolute values for the fp32 accumulation over K terms (doubled
to cover the split-K partial sums).  A dropped term, a wrong index, a
transposed operand or a misplaced tile breaks them by orders of magnitude.
Mirrored elements of A and B must be exactly symmetric."""

import numpy as np
import pytest

from gpu_util import say, to_dev, to_np
from oracle import bf16_round_f32

pytestmark = pytest.mark.gpu

U = 2.0 ** -24  # fp32 unit roundoff


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    assert torch.cuda.is_available()
    return torch


@pytest.fixture(scope="module")
def ctx(torch_mod):
    import muon_step_amd as ms
    c = ms.Context(0)
    yield c
    torch_mod.cuda.synchronize()
    c.close()


# 1 x 1 .. 33 x 65: sub-tile and ragged; 1408 x 2048: the 16B-MoE expert shape
# (padded to 1536); 256 x 2048 (Gram in 4 K ranges), 2048 x 4096 (Gram and A^2
# in 3): long K loops split over several workgroups; 300 x 3000: a split and
# ragged K (Gram in 5).
SHAPES = [(1, 1), (1, 7), (33, 65), (256, 256), (300, 520), (1408, 2048), (256, 2048), (1024, 1536),
          (2048, 4096), (300, 3000)]


def _x(shape, seed):
    s, l = shape
    r = np.random.default_rng(seed)
    x = (r.standard_normal(shape) / np.sqrt(l)).astype(np.float32)
    x.flat[::11] = 0.0   # exact zeros
    return x


def _sym_from(x):
    """A bitwise-symmetric fp32 s x s matrix of O(1) entries."""
    a = (x.astype(np.float64) @ x.astype(np.float64).T).astype(np.float32)
    return np.triu(a) + np.triu(a, 1).T


def _check(got, exact, bound, what):
    err = np.abs(got.astype(np.float64) - exact)
    bad = err > bound
    worst = float(np.max(err / np.maximum(bound, 1e-300)))
    say(f"  {what}: worst error / bound {worst:.3f}")
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of bound, first "
                             f"{[(tuple(i), float(got[tuple(i)]), float(exact[tuple(i)])) for i in idx]}")


def _symmetric_outside_diagonal_blocks(m, what):
    """Elements written as mirrors must equal their source bit for bit; inside the
    32 x 32 blocks on the diagonal both halves are computed directly."""
    s = m.shape[0]
    i, j = np.indices((s, s))
    off = (i // 32) != (j // 32)
    assert np.array_equal(m[off].view(np.uint32), m.T[off].view(np.uint32)), f"{what} not symmetric"


@pytest.mark.parametrize("shape", SHAPES)
def test_gram_stage(ctx, torch_mod, shape):
    import muon_step_amd as ms
    s, l = shape
    x = _x(shape, s * 7 + l)
    out = torch_mod.empty((s, s), dtype=torch_mod.float32, device="cuda")
    ctx.muon_ns_stage(ms.MUON_STAGE_GRAM, out, x=to_dev(x, torch_mod.float32))
    torch_mod.cuda.synchronize()
    got = to_np(out)
    xh = bf16_round_f32(x).astype(np.float64)
    exact = xh @ xh.T
    absprod = np.abs(xh) @ np.abs(xh).T
    say(f"gram {shape}")
    _check(got, exact, 2.0 ** -8 * np.abs(exact) + 2.02 * l * U * absprod + 1e-37, "A")
    _symmetric_outside_diagonal_blocks(got, "A")


@pytest.mark.parametrize("shape", SHAPES)
def test_poly_stage(ctx, torch_mod, shape):
    import muon_step_amd as ms
    s, l = shape
    a_in = _sym_from(_x(shape, s * 5 + l))
    b, c = -4.7750, 2.0315
    out = torch_mod.empty((s, s), dtype=torch_mod.float32, device="cuda")
    ctx.muon_ns_stage(ms.MUON_STAGE_POLY, out, m=to_dev(a_in, torch_mod.float32), b=b, c=c)
    torch_mod.cuda.synchronize()
    got = to_np(out)
    ab = bf16_round_f32(a_in).astype(np.float64)
    a2 = ab @ ab
    exact = b * ab + c * a2
    absprod = np.abs(ab) @ np.abs(ab)
    bound = (2.0 ** -8 * np.abs(exact) + 2.02 * abs(c) * s * U * absprod
             + 2.0 * U * (abs(b) * np.abs(ab) + abs(c) * np.abs(a2)) + 1e-37)
    say(f"poly {shape}")
    _check(got, exact, bound, "B")
    _symmetric_outside_diagonal_blocks(got, "B")


@pytest.mark.parametrize("shape", SHAPES)
def test_apply_stage(ctx, torch_mod, shape):
    import muon_step_amd as ms
    s, l = shape
    x = _x(shape, s * 3 + l)
    b_in = _sym_from(_x((s, max(s, 8)), s + 17)) * np.float32(-1.3)
    a = 3.4445
    out = torch_mod.empty((s, l), dtype=torch_mod.float32, device="cuda")
    ctx.muon_ns_stage(ms.MUON_STAGE_APPLY, out, x=to_dev(x, torch_mod.float32), m=to_dev(b_in, torch_mod.float32),
                      a=a)
    torch_mod.cuda.synchronize()
    got = to_np(out)
    bb = bf16_round_f32(b_in).astype(np.float64)
    xh = bf16_round_f32(x).astype(np.float64)
    x64 = x.astype(np.float64)
    exact = a * x64 + bb @ xh
    absprod = np.abs(bb) @ np.abs(xh)
    # X as hi + residual carries x to 2^-15 (2^-16 unless the residual clamps), and
    # so does the pair X' is stored in; then the fp32 accumulation and the fma
    bound = (2.0 ** -15 * (abs(a) * np.abs(x64) + 1.01 * np.abs(exact)) + 2.02 * s * U * absprod
             + 2.0 * U * np.abs(exact) + 1e-37)
    say(f"apply {shape}")
    _check(got, exact, bound, "X'")
