"""Pins for the oracle's int8 per-row quantizer (CPU only).

Closed forms, brute force over all 255 codes with exact rationals, exact and
near ties, and invariants (error bound, sign symmetry, power-of-two
equivariance, idempotence, row permutation).
"""

from fractions import Fraction

import numpy as np
import pytest

from exact import round_to_f32, round_to_bf16, frac_of_bf16, rne_int
from oracle.bf16 import bf16_to_f64
from oracle.quant import quantize_int8, dequantize_int8
from oracle.matvec import gemv_int8

C_ONES = Fraction(16383, 16384)   # deq of 1.0: q = 127 at s = 129/16384


def test_all_ones_closed_form():
    w = np.ones((3, 64), np.float32)
    q, s = quantize_int8(w)
    assert np.all(s == 0x3C01)                       # bf16(1/127) = 129/16384
    assert frac_of_bf16(int(s[0])) == Fraction(129, 16384)
    assert np.all(q == 127)
    assert np.all(dequantize_int8(q, s) == float(C_ONES))


def test_identity_matvec_closed_form():
    k = 96
    w = np.eye(k, dtype=np.float32)
    q, s = quantize_int8(w)
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(k).astype(np.float32).view(np.uint32) & 0xFFFF0000).view(np.float32)
    x_bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    y = gemv_int8(x_bits, q, s)
    assert np.array_equal(y, x.astype(np.float64) * float(C_ONES))


def _independent_scale(row):
    m = max(abs(Fraction(float(v))) for v in row)
    return round_to_bf16(round_to_f32(m / 127))


@pytest.mark.parametrize("seed,n,k", [(0, 4, 128), (1, 3, 48), (2, 2, 16)])
def test_brute_force_argmin_over_all_codes(seed, n, k):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    for r in range(n):
        s_exact = _independent_scale(w[r])
        assert frac_of_bf16(int(s[r])) == s_exact
        for c in range(k):
            wv = Fraction(float(w[r, c]))
            best = min(range(-127, 128), key=lambda code: (abs(wv - code * s_exact), code % 2))
            assert q[r, c] == best


def test_exact_ties_go_to_even_and_neighbours_round_away_from_tie():
    # a row whose max fixes the scale, plus entries exactly at half-codes
    m = np.float32(1.0)
    s_exact = _independent_scale([m])
    s_val = float(s_exact)
    halves = [k + 0.5 for k in range(0, 126)] + [-(k + 0.5) for k in range(0, 126)]
    ties = np.array([h * s_val for h in halves], np.float32)
    assert all(Fraction(float(t)) == Fraction(h) * s_exact for t, h in zip(ties, halves))  # exact
    up = np.nextafter(ties, np.float32(np.inf))
    down = np.nextafter(ties, np.float32(-np.inf))
    row = np.concatenate([[m], ties, up, down]).astype(np.float32)
    q, s = quantize_int8(row[None, :])
    assert frac_of_bf16(int(s[0])) == s_exact
    n = len(halves)
    got_t, got_u, got_d = q[0, 1:1 + n], q[0, 1 + n:1 + 2 * n], q[0, 1 + 2 * n:]
    for i, h in enumerate(halves):
        lo, hi = int(np.floor(h)), int(np.floor(h)) + 1
        assert got_t[i] == (lo if lo % 2 == 0 else hi)
        assert got_u[i] == hi
        assert got_d[i] == lo


def test_round_half_even_not_away_or_truncate():
    # (k + 1/2) s with k = 2 must give 2, not 3; with k = 3 must give 4
    s_exact = _independent_scale([1.0])
    row = np.array([1.0, 2.5 * float(s_exact), 3.5 * float(s_exact), -2.5 * float(s_exact)], np.float32)
    q, _ = quantize_int8(row[None, :])
    assert q[0].tolist() == [127, 2, 4, -2]


def test_error_bound_code_range_and_extremes():
    rng = np.random.default_rng(4)
    w = (rng.standard_normal((64, 512)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    deq = dequantize_int8(q, s)
    sv = bf16_to_f64(s)[:, None]
    assert np.all(np.abs(w.astype(np.float64) - deq) <= sv / 2)
    assert q.min() >= -127 and q.max() <= 127
    # the largest-magnitude entry of each row always takes code +-127
    idx = np.argmax(np.abs(w), axis=1)
    assert np.all(np.abs(q[np.arange(64), idx]) == 127)


def test_sign_symmetry_and_pow2_equivariance_and_permutation():
    rng = np.random.default_rng(5)
    w = (rng.standard_normal((16, 256)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    qn, sn = quantize_int8(-w)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for j in (-3, 5):
        q2, s2 = quantize_int8((w * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q2, q)
        assert np.array_equal(bf16_to_f64(s2), bf16_to_f64(s) * 2.0 ** j)
    perm = rng.permutation(16)
    qp, sp = quantize_int8(w[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])


def test_idempotent_on_dequantized_weights():
    rng = np.random.default_rng(6)
    w = (rng.standard_normal((8, 320)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    deq32 = dequantize_int8(q, s).astype(np.float32)
    assert np.array_equal(deq32.astype(np.float64), dequantize_int8(q, s))  # exact in fp32
    q2, s2 = quantize_int8(deq32)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_zero_row_and_empty():
    w = np.zeros((2, 32), np.float32)
    w[1, 3] = 0.5
    q, s = quantize_int8(w)
    assert s[0] == 0 and np.all(q[0] == 0)
    assert q[1, 3] == 127 and np.count_nonzero(q[1]) == 1
    q0, s0 = quantize_int8(np.zeros((0, 32), np.float32))
    assert q0.shape == (0, 32) and s0.shape == (0,)


def test_nonfinite_rejected():
    w = np.zeros((1, 16), np.float32)
    w[0, 0] = np.inf
    with pytest.raises(ValueError):
        quantize_int8(w)


def test_scale_matches_exact_rounding_on_many_rows():
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((400, 64)) * rng.uniform(1e-6, 1e3, (400, 1))).astype(np.float32)
    _, s = quantize_int8(w)
    for r in range(400):
        assert frac_of_bf16(int(s[r])) == _independent_scale(w[r])


def test_rne_helper_on_random_quotients():
    rng = np.random.default_rng(8)
    w = (rng.standard_normal((4, 64)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    for r in range(4):
        s_exact = frac_of_bf16(int(s[r]))
        for c in range(64):
            assert q[r, c] == max(-127, min(127, rne_int(Fraction(float(w[r, c])) / s_exact)))
