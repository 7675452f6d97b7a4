"""bf16 encoding for the oracle (test infrastructure only).

The pages fix bf16 as the precision of the unquantized "Base" rows and of the
int4 scales (gittoolsai "gpt-fast" README mirror, benchmark table "基准测试",
rows "Base"); they do not say how values are rounded to it.  The reading
taken is IEEE round-to-nearest-even from fp32, the rounding every bf16
conversion in PyTorch performs.

bf16 is the upper 16 bits of an IEEE binary32.  Rounding keeps those bits
and rounds the dropped 16 bits to nearest, ties to an even kept value.
"""

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_bits(a):
    """fp32 array -> uint32 bit patterns (exact)."""
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def round_f32_to_bf16(a):
    """fp32 values -> bf16 bit patterns (uint16), round to nearest, ties even.

    Worked on the bit pattern: with ``hi`` the kept upper half and ``lo`` the
    dropped lower half, the result is ``hi + 1`` when ``lo > 0x8000`` or when
    ``lo == 0x8000`` and ``hi`` is odd, else ``hi``.  A carry out of the
    mantissa moves into the exponent, which is the correct rounded value
    (up to and including overflow to infinity).  NaN maps to a quiet NaN.
    """
    b = f32_bits(a).astype(np.uint64)
    hi = b >> np.uint64(16)
    lo = b & np.uint64(0xFFFF)
    up = (lo > 0x8000) | ((lo == 0x8000) & ((hi & np.uint64(1)) == 1))
    out = (hi + up.astype(np.uint64)).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    out = np.where(nan, BF16_NAN, out).astype(np.uint16)
    return out


def bf16_to_f32(h):
    """bf16 bit patterns -> fp32 values (exact: bf16 is a subset of fp32)."""
    h = np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return h.view(np.float32)


def bf16_to_f64(h):
    """bf16 bit patterns -> fp64 values (exact)."""
    return bf16_to_f32(h).astype(np.float64)
