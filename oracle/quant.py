"""Weight-only quantizers for the oracle (test infrastructure only).

The pages name two weight-only formats and nothing of their arithmetic:

* int8, one checkpoint per model, fed straight to generation (gittoolsai
  "gpt-fast" README mirror, section "Int8 仅权重量化"; onegen.ai guide,
  "Code Examples / Int8 Quantized Generation");
* int4 with a group-size knob, shown at groups of 32 (same mirror, section
  "Int4 仅权重量化" and the "4-bit (G=32)" rows of the benchmark table;
  awesome-repositories "meta-pytorch/gpt-fast", tag "Grouped Quantization").

The benchmark table's "memory bandwidth" column divided by tokens/s gives the
bytes each format stores per weight: 1 byte plus a bf16 per output row for
int8, 0.625 byte (a 4-bit code plus 2 x 16 bits per group of 32) for int4.
The storage layout here produces exactly those sizes.

Readings taken where the pages are silent (the plainest ones):

* int8: symmetric per output row.  m = max|w| over the row; the fp32
  quotient m/127 (correctly rounded) is rounded to a bf16 scale s; codes are
  q = round-half-even(w / s) of the exact real quotient, clamped to
  [-127, 127].  The stored bf16 s is the one the codes are taken against, so
  |w - q s| <= s/2 holds exactly.  A zero scale gives zero codes.
* int4: asymmetric, G consecutive inputs of one output row per group (G = 32
  unless stated; the group-size knob also takes 64, 128 and 256, which store
  0.5 + 4/G bytes per weight, and its limit G = K, one group per output row:
  per-channel int4, for K a multiple of 32).  The zero z = bf16(min) is the value code 0
  decodes to (a minimum of zero is taken as +0: the minimum of a group holding
  both +0 and -0 is otherwise a matter of comparison order); t = fp32(max - z);
  s = bf16(fp32(t / 15)) when t > 0, else s = 0; codes are
  round-half-even((w - z) / s) of the exact real quotient clamped to [0, 15]
  (all zero when s == 0); w ~ z + q s.
* Packing: byte j of a row holds code 2j in its low nibble and code 2j+1 in
  its high nibble.  Per group the bf16 pair (scale, zero) is stored scale
  first: sz[n][g] = (s, z).
* Non-finite weights are outside the contract: the oracle raises.
"""

import math
from fractions import Fraction

import numpy as np

from .bf16 import round_f32_to_bf16, bf16_to_f32, bf16_to_f64

GROUP = 32
GROUPS = (32, 64, 128, 256)   # group sizes the library supports
INT8_MAX = 127
INT4_MAX = 15

# fp64 quotients are within 2**-44 of the exact ones for every quotient the
# quantizers form (|r| < 2**8 before clamping); a quotient this close to a
# half-integer is re-decided in exact rational arithmetic.
_NEAR_TIE = 2.0 ** -20


def _round_half_even_fraction(f):
    """Nearest integer to an exact rational, ties to the even integer."""
    n = math.floor(f)
    rem = f - n
    half = Fraction(1, 2)
    if rem > half:
        return n + 1
    if rem < half:
        return n
    return n if n % 2 == 0 else n + 1


def round_half_even_quotient(w, z, s):
    """round-half-even((w - z) / s) of the exact real quotient, elementwise.

    w, z, s are fp64 arrays holding exactly the fp32/bf16 values involved
    (broadcastable; s > 0).  The fp64 quotient decides every element that is
    not within 2**-20 of a half-integer; the rest are decided exactly with
    ``fractions.Fraction``.
    """
    w, z, s = np.broadcast_arrays(np.asarray(w, np.float64),
                                  np.asarray(z, np.float64),
                                  np.asarray(s, np.float64))
    r = (w - z) / s
    q = np.rint(r)  # numpy rint rounds half to even
    near = np.abs(r - (np.floor(r) + 0.5)) < _NEAR_TIE
    for idx in zip(*np.nonzero(near)):
        exact = (Fraction(float(w[idx])) - Fraction(float(z[idx]))) / Fraction(float(s[idx]))
        q[idx] = _round_half_even_fraction(exact)
    return q


def _check_finite(w):
    if not np.all(np.isfinite(w)):
        raise ValueError("weights must be finite")


# ----------------------------------------------------------------------------
# int8, per output row


def int8_row_scale(w):
    """bf16 scale per output row: bf16(fp32(max|w| / 127))."""
    w = np.asarray(w, np.float32)
    m = np.max(np.abs(w), axis=-1)
    s32 = (m / np.float32(INT8_MAX)).astype(np.float32)  # IEEE fp32 division
    return round_f32_to_bf16(s32)


def quantize_int8(w):
    """W fp32 [N, K] -> (q int8 [N, K], s bf16 bits uint16 [N])."""
    w = np.asarray(w, np.float32)
    if w.ndim != 2:
        raise ValueError("W must be [N, K]")
    _check_finite(w)
    n, k = w.shape
    s = int8_row_scale(w) if k > 0 else np.zeros(n, np.uint16)
    sv = bf16_to_f64(s)
    q = np.zeros((n, k), np.float64)
    rows = sv > 0
    if k > 0 and rows.any():
        q[rows] = round_half_even_quotient(w[rows].astype(np.float64), 0.0,
                                           sv[rows][:, None])
    q = np.clip(q, -INT8_MAX, INT8_MAX)
    return q.astype(np.int8), s


def dequantize_int8(q, s):
    """deq[n, k] = q[n, k] * s[n], exact in fp64."""
    return np.asarray(q, np.float64) * bf16_to_f64(s)[..., None]


# ----------------------------------------------------------------------------
# int4, groups of G inputs (32 by default), bf16 scale and zero


def int4_scale_zero(w, group=GROUP):
    """Per-group (s, z) bf16 bit patterns, each [N, K/group].

    z = bf16(min), t = fp32(max - z), s = bf16(fp32(t / 15)) if t > 0 else 0.
    A zero minimum is +0 (adding +0 maps -0 to +0 and changes nothing else).
    """
    w = np.asarray(w, np.float32)
    n, k = w.shape
    g = w.reshape(n, k // group, group)
    mn = (g.min(axis=2) + np.float32(0.0)).astype(np.float32)
    mx = g.max(axis=2)
    z = round_f32_to_bf16(mn)
    t = (mx - bf16_to_f32(z)).astype(np.float32)          # IEEE fp32 subtraction
    s32 = (t / np.float32(INT4_MAX)).astype(np.float32)    # IEEE fp32 division
    s = np.where(t > 0, round_f32_to_bf16(s32), np.uint16(0)).astype(np.uint16)
    return s, z


def int4_codes(w, s, z, group=GROUP):
    """Codes q[n, k] in [0, 15] and the count of codes the clamp changed."""
    w = np.asarray(w, np.float32)
    n, k = w.shape
    g = w.reshape(n, k // group, group).astype(np.float64)
    sv = bf16_to_f64(s)[..., None]
    zv = bf16_to_f64(z)[..., None]
    q = np.zeros(g.shape, np.float64)
    sel = sv[..., 0] > 0
    if sel.any():
        q[sel] = round_half_even_quotient(g[sel], zv[sel], sv[sel])
    clamped = int(np.count_nonzero((q < 0) | (q > INT4_MAX)))
    q = np.clip(q, 0, INT4_MAX)
    return q.reshape(n, k).astype(np.uint8), clamped


def pack_int4(q):
    """Codes [N, K] (0..15) -> bytes [N, K/2]: low nibble = even k."""
    q = np.asarray(q, np.uint8)
    return (q[:, 0::2] | (q[:, 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed):
    """Bytes [N, K/2] -> codes [N, K] (inverse of ``pack_int4``)."""
    p = np.asarray(packed, np.uint8)
    n, h = p.shape
    q = np.empty((n, 2 * h), np.uint8)
    q[:, 0::2] = p & 0x0F
    q[:, 1::2] = p >> 4
    return q


def quantize_int4(w, group=GROUP, return_clamped=False):
    """W fp32 [N, K] (K % group == 0) -> (packed u8 [N, K/2], sz u16 [N, K/group, 2]).

    group is one of ``GROUPS`` or K itself (one group per row, K a positive
    multiple of 32).  With ``return_clamped`` also returns how many codes the
    [0, 15] clamp changed (never any for groups that span zero; only a group
    of one sign whose range is tiny next to its magnitude can clamp at code 0).
    """
    w = np.asarray(w, np.float32)
    if w.ndim != 2:
        raise ValueError("W must be [N, K]")
    k = w.shape[1]
    per_row = group == k and k > 0 and k % GROUP == 0
    if group not in GROUPS and not per_row:
        raise ValueError(f"group must be one of {GROUPS} or K (a multiple of {GROUP})")
    if k % group != 0:
        raise ValueError(f"W must be [N, K] with K a multiple of {group}")
    _check_finite(w)
    n, k = w.shape
    s, z = int4_scale_zero(w, group)
    q, clamped = int4_codes(w, s, z, group)
    packed = pack_int4(q)
    sz = np.stack([s, z], axis=-1).astype(np.uint16)
    if return_clamped:
        return packed, sz, clamped
    return packed, sz


def dequantize_int4(packed, sz):
    """deq[n, k] = z[n, g] + q[n, k] * s[n, g] with g = k // G, exact in fp64;
    the group size G is K over the number of (s, z) pairs per row.  K = 0
    (no groups) is the empty [n, 0] matrix."""
    q = unpack_int4(packed).astype(np.float64)
    n, k = q.shape
    groups = sz.shape[1]
    if k == 0 and groups == 0:
        return q
    if groups == 0 or k % groups:
        raise ValueError("sz must hold K/G (scale, zero) pairs per row")
    s = bf16_to_f64(sz[..., 0])
    z = bf16_to_f64(sz[..., 1])
    g = q.reshape(n, groups, k // groups)
    return (z[..., None] + g * s[..., None]).reshape(n, k)


# The G = 32 names: the benchmark table's "4-bit (G=32)" format.
def quantize_int4g32(w, return_clamped=False):
    """``quantize_int4`` with groups of 32."""
    return quantize_int4(w, GROUP, return_clamped)


def int4g32_scale_zero(w):
    return int4_scale_zero(w, GROUP)


def int4g32_codes(w, s, z):
    return int4_codes(w, s, z, GROUP)


dequantize_int4g32 = dequantize_int4
