"""Pins for the oracle's dequantized matvec (CPU only).

Exact rational products on tiny shapes, an explicit row-by-row loop (catches a
transposed operand), the per-group decomposition the kernels use, and the
speculative-verify rows.
"""

from fractions import Fraction

import numpy as np
import pytest

from exact import frac_of_bf16
from oracle.bf16 import round_f32_to_bf16
from oracle.quant import quantize_int8, quantize_int4g32, unpack_int4
from oracle.matvec import gemv_bf16, gemv_int8, gemv_int4g32, gemm_small_m, gemv_int8_f64x, gemm_small_m_int8


def _bits(rng, shape):
    return round_f32_to_bf16(rng.standard_normal(shape).astype(np.float32))


def test_int4_exact_rational_and_group_decomposition():
    rng = np.random.default_rng(21)
    n, k = 3, 96
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    packed, sz = quantize_int4g32(w)
    x = _bits(rng, k)
    y = gemv_int4g32(x, packed, sz)
    q = unpack_int4(packed)
    xf = [frac_of_bf16(int(v)) for v in x]
    for r in range(n):
        total = Fraction(0)
        for g in range(k // 32):
            s = frac_of_bf16(int(sz[r, g, 0]))
            z = frac_of_bf16(int(sz[r, g, 1]))
            xs = sum(xf[32 * g:32 * g + 32], Fraction(0))
            qx = sum((int(q[r, c]) * xf[c] for c in range(32 * g, 32 * g + 32)), Fraction(0))
            total += s * qx + z * xs
        assert abs(Fraction(float(y[r])) - total) <= abs(total) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 30)


def test_int8_exact_rational_rows_not_columns():
    rng = np.random.default_rng(22)
    n, k = 5, 48                                  # non-square: a transpose cannot pass
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    x = _bits(rng, k)
    y = gemv_int8(x, q, s)
    assert y.shape == (n,)
    xf = [frac_of_bf16(int(v)) for v in x]
    for r in range(n):
        want = frac_of_bf16(int(s[r])) * sum((int(q[r, c]) * xf[c] for c in range(k)), Fraction(0))
        assert abs(Fraction(float(y[r])) - want) <= abs(want) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 30)


def test_bf16_exact_rational():
    rng = np.random.default_rng(23)
    n, k = 4, 40
    wb = _bits(rng, (n, k))
    x = _bits(rng, k)
    y = gemv_bf16(x, wb)
    for r in range(n):
        want = sum((frac_of_bf16(int(wb[r, c])) * frac_of_bf16(int(x[c])) for c in range(k)), Fraction(0))
        assert abs(Fraction(float(y[r])) - want) <= abs(want) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 30)


def test_bf16_identity_and_ones():
    k = 64
    x = _bits(np.random.default_rng(24), k)
    eye = round_f32_to_bf16(np.eye(k, dtype=np.float32))
    assert np.array_equal(gemv_bf16(x, eye), frac_to_f64(x))
    ones = round_f32_to_bf16(np.ones((3, k), np.float32))
    assert np.allclose(gemv_bf16(x, ones), frac_to_f64(x).sum(), rtol=0, atol=1e-12)


def frac_to_f64(bits):
    return np.array([float(frac_of_bf16(int(v))) for v in bits])


def test_small_m_rows_are_independent_gemvs():
    rng = np.random.default_rng(25)
    w = (rng.standard_normal((7, 128)) * 0.015).astype(np.float32)
    packed, sz = quantize_int4g32(w)
    x = _bits(rng, (5, 128))
    y = gemm_small_m(x, packed, sz)
    assert y.shape == (5, 7)
    for m in range(5):
        assert np.array_equal(y[m], gemv_int4g32(x[m], packed, sz))
    # a permutation of token rows permutes output rows
    perm = [3, 0, 4, 1, 2]
    assert np.array_equal(gemm_small_m(x[perm], packed, sz), y[perm])


def test_f64_activation_path_matches_bf16_path_on_bf16_values():
    rng = np.random.default_rng(26)
    w = (rng.standard_normal((6, 64)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    x = _bits(rng, 64)
    assert np.array_equal(gemv_int8_f64x(frac_to_f64(x), q, s), gemv_int8(x, q, s))


def test_empty_k_and_n():
    q = np.zeros((3, 0), np.int8)
    s = np.zeros(3, np.uint16)
    assert np.array_equal(gemv_int8(np.zeros(0, np.uint16), q, s), np.zeros(3))
    packed = np.zeros((0, 16), np.uint8)
    sz = np.zeros((0, 1, 2), np.uint16)
    assert gemv_int4g32(np.zeros(32, np.uint16), packed, sz).shape == (0,)


def test_int8_small_m_exact_rational_and_rows():
    """M token rows through an int8 linear: y[m, n] = s[n] sum_k x[m, k] q[n, k]
    exactly (non-square M, N, K: a swapped index fails), each row equal to
    the one-token product, and permuted token rows give permuted outputs."""
    rng = np.random.default_rng(26)
    m, n, k = 3, 5, 48
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    q, s = quantize_int8(w)
    x = _bits(rng, (m, k))
    y = gemm_small_m_int8(x, q, s)
    assert y.shape == (m, n)
    for t in range(m):
        xf = [frac_of_bf16(int(v)) for v in x[t]]
        for r in range(n):
            want = frac_of_bf16(int(s[r])) * sum((int(q[r, c]) * xf[c] for c in range(k)), Fraction(0))
            assert abs(Fraction(float(y[t, r])) - want) <= abs(want) * Fraction(1, 10 ** 14) + Fraction(1, 10 ** 30)
        assert np.array_equal(y[t], gemv_int8(x[t], q, s))
    perm = [2, 0, 1]
    assert np.array_equal(gemm_small_m_int8(x[perm], q, s), y[perm])
    with pytest.raises(ValueError):
        gemm_small_m_int8(x[0], q, s)
