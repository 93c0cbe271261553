"""Kernel unit tests of the three bf16 Newton-Schulz products (one step is
X <- a X + b A X + c A^2 X with A = X X^T, DeepSeek-V4 book ch. 6 section 3),
each run alone through the muon_ns_stage hook exactly as muon_step runs it for
one matrix of that shape (same tiles, same split of long K loops), and compared
element by element with fp64 products of the *same* bf16 operands:

  GRAM   A = bf16(X_hi X_hi^T)            X_hi the pair's hi of X
  POLY   B = bf16(b A + c A A)            A given, rounded to bf16
  APPLY  X' = a X + B X_hi                B rounded to bf16, X kept as hi + residual

The bounds are those of the arithmetic: the final rounding to bf16 (half an
ulp of an 8-bit significand: 2^-8 relative) or to the hi + residual pair
(2^-16 relative, on the way in and out), plus K 2^-24 times the
product of the absolute values for the fp32 accumulation over K terms (doubled
to cover the split-K partial sums).  A dropped term, a wrong index, a
transposed operand or a misplaced tile breaks them by orders of magnitude.
Mirrored elements of A and B must be exactly symmetric."""

import numpy as np
import pytest

from gpu_util import pair_hi, say, to_dev, to_np
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
# ragged K (Gram in 5); 4352^2: the apply's 33 tiles past its first wave split
# over K (7 ranges) and reduced with the a X term.
SHAPES = [(1, 1), (1, 7), (33, 65), (256, 256), (300, 520), (1408, 2048), (256, 2048), (1024, 1536),
          (2048, 4096), (300, 3000), (4352, 4352)]


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
    xh = pair_hi(x).astype(np.float64)
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
    xh = pair_hi(x).astype(np.float64)
    x64 = x.astype(np.float64)
    exact = a * x64 + bb @ xh
    absprod = np.abs(bb) @ np.abs(xh)
    # X as hi + residual carries x to 2^-16 of its magnitude, and so does the pair
    # X' is stored in; then the fp32 accumulation and the fma
    bound = (1.01 * 2.0 ** -16 * (abs(a) * np.abs(x64) + np.abs(exact)) + 2.02 * s * U * absprod
             + 2.0 * U * np.abs(exact) + 1e-37)
    say(f"apply {shape}")
    _check(got, exact, bound, "X'")


def _pair_round_trip(x):
    """Emulated decode(encode(x)) of the pair codec, on fp32 bit patterns: hi = top
    16 bits of b + 0x8080 (b capped at 0x7fff7f7f, the sum saturating), residual
    = bits 8..15 of b + 0x80 read as a signed byte, value (hi << 16) + (q << 8)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.int32).astype(np.int64)
    y = np.minimum((np.minimum(b, 0x7FFF7F7F) & 0xFFFFFFFF) + 0x8080, 0xFFFFFFFF)
    hi = y >> 16
    q = (((y >> 8) & 0xFF) ^ 0x80).astype(np.uint8).view(np.int8).astype(np.int64)
    return ((((hi << 16) + (q << 8)) & 0xFFFFFFFF).astype(np.uint32)).view(np.float32)


def test_pair_codec_round_trip(ctx, torch_mod):
    """X' = 1 X + 0 X_hi through the apply stage returns, for every finite input
    whose hi stays finite, the decode of its encoding in the (hi, residual) pair,
    bit for bit (-0 comes back as +0: the product term is +0).  The inputs cover
    zeros, subnormals, every exponent, and low halves of the bit pattern at the
    rounding boundaries of hi (0x7f80, 0x8000) and of the residual (0x7f, 0x80)."""
    import muon_step_amd as ms
    r = np.random.default_rng(77)
    pats = [0x00000000, 0x80000000, 0x00000001, 0x80000001, 0x000000FF, 0x00007F80, 0x00008000,
            0x007FFFFF, 0x807FFFFF, 0x00800000, 0x7F7F7F7F, 0xFF7F7F7F]
    for e in range(1, 255, 2):
        for low in (0x0000, 0x007F, 0x0080, 0x00FF, 0x7F7F, 0x7F80, 0x7FFF, 0x8000, 0x8001, 0x807F, 0x8080, 0xFFFF):
            m = (int(r.integers(0, 128)) << 16) | low
            for sign in (0, 1):
                pats.append((sign << 31) | (e << 23) | m)
    pats = np.array(pats, dtype=np.uint64)
    pats = pats[(pats & 0x7FFFFFFF) < 0x7F7F7F80]          # hi stays finite (0 x inf would be NaN)
    s, l = 32, 128
    rand = (r.standard_normal(s * l - pats.size) * np.exp2(r.integers(-60, 60, s * l - pats.size))).astype(np.float32)
    x = np.concatenate([pats.astype(np.uint32).view(np.float32), rand]).reshape(s, l)
    out = torch_mod.empty((s, l), dtype=torch_mod.float32, device="cuda")
    ctx.muon_ns_stage(ms.MUON_STAGE_APPLY, out, x=to_dev(x, torch_mod.float32),
                      m=to_dev(np.zeros((s, s), np.float32), torch_mod.float32), a=1.0)
    torch_mod.cuda.synchronize()
    got = to_np(out)
    want = _pair_round_trip(x)
    want = np.where(want == 0, np.float32(0.0), want)       # -0 + (+0) = +0
    say(f"pair codec: {x.size} values")
    bad = got.view(np.uint32) != want.view(np.uint32)
    if np.any(bad):
        i = np.argwhere(bad)[:5]
        raise AssertionError(f"{int(bad.sum())} values differ, first "
                             f"{[(hex(int(x.view(np.uint32)[tuple(k)])), hex(int(got.view(np.uint32)[tuple(k)])), hex(int(want.view(np.uint32)[tuple(k)]))) for k in i]}")
    rel = np.abs(got.astype(np.float64) - x) / np.maximum(np.abs(x.astype(np.float64)), 1e-300)
    normal = np.abs(x) >= np.finfo(np.float32).tiny
    assert np.max(rel[normal]) <= 2.0 ** -16 * (1 + 2.0 ** -7)
