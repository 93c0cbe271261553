"""bfloat16 rounding for the oracle (test infrastructure only).

bfloat16 is the upper 16 bits of an IEEE binary32.  A float32 value is
rounded to it with round-to-nearest, ties to even (the only rounding mode the
Muon step uses on its hot path); NaN stays NaN (quiet, sign kept), infinities
stay infinite and values past the largest finite bfloat16 round to infinity.
"""

import numpy as np


def f32_to_bf16_bits(x):
    """float32 array -> uint16 array of bfloat16 bit patterns (RNE)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    nan = np.isnan(x)
    # Add half an ulp of the kept part, plus one if the kept part is odd, then truncate.
    keep_lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + keep_lsb) >> np.uint64(16)
    r = r.astype(np.uint32)
    quiet = ((u >> np.uint64(16)).astype(np.uint32) | np.uint32(0x0040))
    r = np.where(nan, quiet, r)
    return (r & np.uint32(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(b):
    """uint16 bfloat16 bit patterns -> float32 (exact widening)."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round_f32(x):
    """Round float32 values to the nearest bfloat16 and return them as float32."""
    return bf16_bits_to_f32(f32_to_bf16_bits(x))
