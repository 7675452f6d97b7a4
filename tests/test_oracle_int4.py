"""Pins for the oracle's int4 G=32 asymmetric quantizer (CPU only)."""

from fractions import Fraction

import numpy as np
import pytest

from exact import round_to_f32, round_to_bf16, frac_of_bf16
from oracle.bf16 import bf16_to_f64
from oracle.quant import (quantize_int4g32, dequantize_int4g32, unpack_int4, pack_int4)
from oracle.matvec import gemv_int4g32

C_ID = Fraction(2055, 2048)   # deq of 1.0 in a group {0 x 31, 1}: z = 0, s = 137/2048, q = 15


def _independent_scale_zero(group):
    vals = [Fraction(float(v)) for v in group]
    z = round_to_bf16(min(vals))
    t = round_to_f32(max(vals) - z)
    s = round_to_bf16(round_to_f32(t / 15)) if t > 0 else Fraction(0)
    return s, z


def test_identity_closed_form():
    k = 128
    w = np.eye(k, dtype=np.float32)
    packed, sz = quantize_int4g32(w)
    s = sz[..., 0]
    z = sz[..., 1]
    rows = np.arange(k)
    own = rows // 32
    assert np.all(s[rows, own] == 0x3D89)            # bf16(1/15) = 137/2048
    assert frac_of_bf16(0x3D89) == Fraction(137, 2048)
    assert np.all(z == 0)
    other = np.ones_like(s, bool)
    other[rows, own] = False
    assert np.all(s[other] == 0)                      # all-zero groups: scale 0
    q = unpack_int4(packed)
    assert np.all(q[rows, rows] == 15) and np.count_nonzero(q) == k
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(k).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    y = gemv_int4g32((x.view(np.uint32) >> 16).astype(np.uint16), packed, sz)
    assert np.array_equal(y, x.astype(np.float64) * float(C_ID))


def test_all_ones_closed_form():
    w = np.ones((2, 64), np.float32)
    packed, sz = quantize_int4g32(w)
    assert np.all(sz[..., 0] == 0) and np.all(sz[..., 1] == 0x3F80)   # s = 0, z = 1
    assert np.all(packed == 0)
    x = np.arange(64, dtype=np.float32)                                  # bf16-exact ints
    y = gemv_int4g32((x.view(np.uint32) >> 16).astype(np.uint16), packed, sz)
    assert np.array_equal(y, np.full(2, x.sum(), np.float64))


@pytest.mark.parametrize("seed,n,k", [(0, 4, 128), (1, 2, 64), (2, 3, 32)])
def test_brute_force_argmin_over_all_codes(seed, n, k):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    packed, sz = quantize_int4g32(w)
    q = unpack_int4(packed)
    for r in range(n):
        for g in range(k // 32):
            grp = w[r, 32 * g:32 * g + 32]
            s_ex, z_ex = _independent_scale_zero(grp)
            assert frac_of_bf16(int(sz[r, g, 0])) == s_ex
            assert frac_of_bf16(int(sz[r, g, 1])) == z_ex
            for c in range(32):
                wv = Fraction(float(grp[c]))
                best = min(range(16), key=lambda code: (abs(wv - (z_ex + code * s_ex)), code % 2))
                assert q[r, 32 * g + c] == best


def test_exact_ties_even_and_neighbours():
    # group: min 0 -> z = 0; max 1 -> s = 137/2048; then exact half-codes
    s_ex = Fraction(137, 2048)
    halves = [k + 0.5 for k in range(0, 10)]
    ties = [float(h * s_ex) for h in halves]
    assert all(Fraction(np.float32(t).item()) == Fraction(h) * s_ex for t, h in zip(ties, halves))
    base = np.zeros(32, np.float32)
    base[0], base[1] = 0.0, 1.0
    base[2:12] = ties
    up = base.copy()
    up[2:12] = np.nextafter(np.float32(ties), np.float32(np.inf))
    down = base.copy()
    down[2:12] = np.nextafter(np.float32(ties), np.float32(-np.inf))
    packed, sz = quantize_int4g32(np.stack([base, up, down]))
    assert np.all(sz[:, 0, 0] == 0x3D89) and np.all(sz[:, 0, 1] == 0)
    q = unpack_int4(packed)
    for i, h in enumerate(halves):
        lo, hi = int(h - 0.5), int(h + 0.5)
        assert q[0, 2 + i] == (lo if lo % 2 == 0 else hi)
        assert q[1, 2 + i] == hi
        assert q[2, 2 + i] == lo


def test_error_bound_ranges_and_extreme_codes():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((48, 512)) * 0.02).astype(np.float32)
    packed, sz, clamped = quantize_int4g32(w, return_clamped=True)
    assert clamped == 0
    deq = dequantize_int4g32(packed, sz)
    s = np.repeat(bf16_to_f64(sz[..., 0]), 32, axis=1)
    assert np.all(np.abs(w.astype(np.float64) - deq) <= s / 2)
    q = unpack_int4(packed).reshape(48, 16, 32)
    gw = w.reshape(48, 16, 32)
    # the group minimum takes code 0 and the group maximum code 15
    assert np.all(np.take_along_axis(q, gw.argmin(axis=2)[..., None], 2) == 0)
    assert np.all(np.take_along_axis(q, gw.argmax(axis=2)[..., None], 2) == 15)


def test_zero_is_the_bf16_group_minimum_not_an_integer_zero_point():
    rng = np.random.default_rng(13)
    w = (rng.standard_normal((4, 64)) * 0.02 + 0.05).astype(np.float32)   # one-signed groups
    _, sz = quantize_int4g32(w)
    for r in range(4):
        for g in range(2):
            assert frac_of_bf16(int(sz[r, g, 1])) == round_to_bf16(Fraction(float(w[r, 32 * g:32 * g + 32].min())))


def test_pow2_equivariance_idempotence_permutation():
    rng = np.random.default_rng(14)
    w = (rng.standard_normal((12, 256)) * 0.02).astype(np.float32)
    packed, sz = quantize_int4g32(w)
    for j in (-4, 6):
        p2, sz2 = quantize_int4g32((w * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(p2, packed)
        assert np.array_equal(bf16_to_f64(sz2), bf16_to_f64(sz) * 2.0 ** j)
    deq = dequantize_int4g32(packed, sz)
    deq32 = deq.astype(np.float32)
    assert np.array_equal(deq32.astype(np.float64), deq)                  # exact in fp32
    p3, sz3 = quantize_int4g32(deq32)
    assert np.array_equal(p3, packed) and np.array_equal(sz3, sz)
    perm = rng.permutation(12)
    pp, szp = quantize_int4g32(w[perm])
    assert np.array_equal(pp, packed[perm]) and np.array_equal(szp, sz[perm])


def test_nibble_order_and_pack_roundtrip():
    q = np.array([[1, 2, 3, 4] + [0] * 28], np.uint8)
    p = pack_int4(q)
    assert p[0, 0] == 0x21 and p[0, 1] == 0x43        # low nibble = even k
    rng = np.random.default_rng(15)
    q = rng.integers(0, 16, (5, 96)).astype(np.uint8)
    assert np.array_equal(unpack_int4(pack_int4(q)), q)


def test_constant_and_degenerate_groups():
    w = np.zeros((3, 64), np.float32)
    w[0, :32] = 0.3                     # constant group, bf16(0.3) rounds away from 0.3
    w[1, :32] = 0.5                     # bf16-exact constant
    w[2, 5] = -1e-3                     # one nonzero in a zero group
    packed, sz = quantize_int4g32(w)
    deq = dequantize_int4g32(packed, sz)
    assert np.all(deq[1, :32] == 0.5) and sz[1, 0, 0] == 0
    assert np.all(deq[:, 32:] == 0)
    assert np.all(np.abs(deq[0, :32] - np.float64(np.float32(0.3))) <= 2.0 ** -9)
    s = bf16_to_f64(sz[2, 0, 0])
    assert abs(deq[2, 5] + 1e-3) <= s / 2 + 1e-12 and np.all(np.abs(deq[2, :32]) <= 1e-3 + s)


def test_shape_checks():
    with pytest.raises(ValueError):
        quantize_int4g32(np.zeros((2, 48), np.float32))
    w = np.zeros((1, 32), np.float32)
    w[0, 0] = np.nan
    with pytest.raises(ValueError):
        quantize_int4g32(w)


def test_clamp_is_reported_for_tight_one_signed_groups():
    # range tiny next to magnitude: bf16(min) lies above min by more than s/2
    w = np.full((1, 32), 1.0, np.float32)
    w[0, 0] = np.float32(1.0) - np.float32(2.0 ** -12)
    w[0, 1] = np.float32(1.0) + np.float32(2.0 ** -12)
    packed, sz, clamped = quantize_int4g32(w, return_clamped=True)
    q = unpack_int4(packed)
    assert q.min() >= 0 and q.max() <= 15
    assert clamped >= 1


# ----------------------------------------------------------------------------
# The group-size knob: G = 64, 128, 256 (the pages' int4 format takes a group
# size; the benchmark table shows G = 32).  The same readings per group of G.

from oracle.quant import quantize_int4, dequantize_int4, GROUPS
from oracle.matvec import gemv_int4

LARGE = [g for g in GROUPS if g != 32]


@pytest.mark.parametrize("group", LARGE)
def test_groups_brute_force_argmin_over_all_codes(group):
    rng = np.random.default_rng(group)
    n, k = 3, 2 * group
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    packed, sz = quantize_int4(w, group)
    assert packed.shape == (n, k // 2) and sz.shape == (n, k // group, 2)
    q = unpack_int4(packed)
    for r in range(n):
        for g in range(k // group):
            grp = w[r, group * g:group * (g + 1)]
            s_ex, z_ex = _independent_scale_zero(grp)
            assert frac_of_bf16(int(sz[r, g, 0])) == s_ex
            assert frac_of_bf16(int(sz[r, g, 1])) == z_ex
            for c in range(0, group, 7):
                wv = Fraction(float(grp[c]))
                best = min(range(16), key=lambda code: (abs(wv - (z_ex + code * s_ex)), code % 2))
                assert q[r, group * g + c] == best


@pytest.mark.parametrize("group", LARGE)
def test_groups_span_group_inputs_not_32(group):
    """A row whose 32-input blocks have disjoint ranges: with groups of G the
    (scale, zero) of each group covers all G inputs (min of the first block,
    max of the last), which no group of 32 reproduces."""
    blocks = group // 32
    w = np.concatenate([np.linspace(b, b + 0.5, 32, dtype=np.float32) for b in range(blocks)])[None, :]
    packed, sz = quantize_int4(w, group)
    assert sz.shape == (1, 1, 2)
    s_ex, z_ex = _independent_scale_zero(w[0])
    assert z_ex == 0 and frac_of_bf16(int(sz[0, 0, 1])) == 0
    assert frac_of_bf16(int(sz[0, 0, 0])) == s_ex == round_to_bf16(round_to_f32(Fraction(blocks - 0.5) / 15))
    q = unpack_int4(packed)
    assert q[0, 0] == 0 and q[0, -1] == 15
    p32, sz32 = quantize_int4(w, 32)
    assert sz32.shape == (1, blocks, 2) and not np.array_equal(unpack_int4(p32), q)


@pytest.mark.parametrize("group", LARGE)
def test_groups_error_bound_extremes_and_identity(group):
    rng = np.random.default_rng(100 + group)
    w = (rng.standard_normal((16, 4 * group)) * 0.02).astype(np.float32)
    packed, sz, clamped = quantize_int4(w, group, return_clamped=True)
    assert clamped == 0
    deq = dequantize_int4(packed, sz)
    s = np.repeat(bf16_to_f64(sz[..., 0]), group, axis=1)
    assert np.all(np.abs(w.astype(np.float64) - deq) <= s / 2)
    q = unpack_int4(packed).reshape(16, 4, group)
    gw = w.reshape(16, 4, group)
    assert np.all(np.take_along_axis(q, gw.argmin(axis=2)[..., None], 2) == 0)
    assert np.all(np.take_along_axis(q, gw.argmax(axis=2)[..., None], 2) == 15)
    # identity: every group holds at most one 1, so s = bf16(1/15), z = 0 as for G = 32
    k = 2 * group
    pe, sze = quantize_int4(np.eye(k, dtype=np.float32), group)
    rows = np.arange(k)
    assert np.all(sze[rows, rows // group, 0] == 0x3D89) and np.all(sze[..., 1] == 0)
    x = (rng.standard_normal(k).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    y = gemv_int4((x.view(np.uint32) >> 16).astype(np.uint16), pe, sze)
    assert np.array_equal(y, x.astype(np.float64) * float(C_ID))


@pytest.mark.parametrize("group", LARGE)
def test_groups_matvec_exact_rational(group):
    rng = np.random.default_rng(200 + group)
    n, k = 3, 2 * group
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    packed, sz = quantize_int4(w, group)
    x = (rng.standard_normal(k).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = gemv_int4(x, packed, sz)
    q = unpack_int4(packed)
    xf = [frac_of_bf16(int(v)) for v in x]
    for r in range(n):
        total = Fraction(0)
        for g in range(k // group):
            s = frac_of_bf16(int(sz[r, g, 0]))
            z = frac_of_bf16(int(sz[r, g, 1]))
            lo, hi = group * g, group * (g + 1)
            total += s * sum((int(q[r, c]) * xf[c] for c in range(lo, hi)), Fraction(0)) + z * sum(xf[lo:hi], Fraction(0))
        assert abs(Fraction(float(y[r])) - total) <= abs(total) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 30)


def test_group_argument_checks():
    with pytest.raises(ValueError):
        quantize_int4(np.zeros((2, 64), np.float32), 48)
    with pytest.raises(ValueError):
        quantize_int4(np.zeros((2, 96), np.float32), 64)


def test_empty_rows_dequantize_to_empty():
    """K = 0: no groups, an empty [N, 0] matrix, and every output of the
    matvec is the empty sum 0."""
    from oracle.quant import dequantize_int4
    from oracle.matvec import gemv_int4
    p = np.zeros((7, 0), np.uint8)
    sz = np.zeros((7, 0, 2), np.uint16)
    assert dequantize_int4(p, sz).shape == (7, 0)
    assert np.array_equal(gemv_int4(np.zeros(0, np.uint16), p, sz), np.zeros(7))


# Per-channel int4: the group-size knob at its limit G = K (one group per row).

@pytest.mark.parametrize("k", [96, 288, 32])
def test_per_channel_brute_force_argmin_over_all_codes(k):
    rng = np.random.default_rng(300 + k)
    w = (rng.standard_normal((3, k)) * 0.02).astype(np.float32)
    packed, sz = quantize_int4(w, k)
    assert packed.shape == (3, k // 2) and sz.shape == (3, 1, 2)
    q = unpack_int4(packed)
    for r in range(3):
        s_ex, z_ex = _independent_scale_zero(w[r])
        assert frac_of_bf16(int(sz[r, 0, 0])) == s_ex
        assert frac_of_bf16(int(sz[r, 0, 1])) == z_ex
        for c in range(0, k, 5):
            wv = Fraction(float(w[r, c]))
            best = min(range(16), key=lambda code: (abs(wv - (z_ex + code * s_ex)), code % 2))
            assert q[r, c] == best


def test_per_channel_one_scale_zero_spans_the_row():
    """Blocks of 32 with disjoint ranges 0..0.5, 1..1.5, 2..2.5: the row's one
    (scale, zero) is (bf16(fp32(2.5 / 15)), 0); the first input takes code 0 and
    the last code 15; every input is within s/2 of its decoded value."""
    w = np.concatenate([np.linspace(b, b + 0.5, 32, dtype=np.float32) for b in range(3)])[None, :]
    packed, sz, clamped = quantize_int4(w, 96, return_clamped=True)
    assert clamped == 0 and sz.shape == (1, 1, 2)
    assert frac_of_bf16(int(sz[0, 0, 0])) == round_to_bf16(round_to_f32(Fraction(5, 2) / 15))
    assert sz[0, 0, 1] == 0
    q = unpack_int4(packed)
    assert q[0, 0] == 0 and q[0, -1] == 15
    deq = dequantize_int4(packed, sz)
    assert np.all(np.abs(w.astype(np.float64) - deq) <= bf16_to_f64(sz[0, 0, 0]) / 2)


def test_per_channel_matvec_exact_rational():
    rng = np.random.default_rng(400)
    n, k = 4, 160
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    packed, sz = quantize_int4(w, k)
    x = (rng.standard_normal(k).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    y = gemv_int4(x, packed, sz)
    q = unpack_int4(packed)
    xf = [frac_of_bf16(int(v)) for v in x]
    for r in range(n):
        s = frac_of_bf16(int(sz[r, 0, 0]))
        z = frac_of_bf16(int(sz[r, 0, 1]))
        total = s * sum((int(q[r, c]) * xf[c] for c in range(k)), Fraction(0)) + z * sum(xf, Fraction(0))
        assert abs(Fraction(float(y[r])) - total) <= abs(total) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 30)


def test_per_channel_argument_checks():
    with pytest.raises(ValueError):
        quantize_int4(np.zeros((2, 48), np.float32), 48)      # K not a multiple of 32
    with pytest.raises(ValueError):
        quantize_int4(np.zeros((2, 192), np.float32), 96)     # neither a listed size nor K
    with pytest.raises(ValueError):
        quantize_int4(np.zeros((2, 0), np.float32), 0)


@pytest.mark.parametrize("group", [32, 64, 96])
def test_zero_minimum_is_positive_zero(group):
    """A group whose minimum is zero stores z = +0 (bits 0x0000) whether the
    zeros are +0, -0 or both, in any order; codes and scale are unchanged by
    the sign of a zero."""
    base = np.linspace(0.0, 1.0, group, dtype=np.float32)
    rows = []
    for pattern in ([0.0], [-0.0], [0.0, -0.0], [-0.0, 0.0]):
        r = base.copy()
        r[:len(pattern)] = np.array(pattern, np.float32)
        rows.append(r[::-1].copy())
        rows.append(r)
    w = np.stack(rows)
    packed, sz = quantize_int4(w, group)
    assert np.all(sz[:, 0, 1] == 0)
    assert np.all(sz[:, 0, 0] == sz[0, 0, 0])
    q = unpack_int4(packed)
    for i in range(0, len(rows), 2):
        assert np.array_equal(q[i], q[1][::-1]) and np.array_equal(q[i + 1], q[1])
