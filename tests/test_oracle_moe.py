"""Pins for the oracle's top-2 MoE (CPU only)."""

import itertools
import math

import numpy as np
import pytest

from oracle.bf16 import round_f32_to_bf16, bf16_to_f64
from oracle.quant import quantize_int8
from oracle.moe import route_top2, moe_top2, silu

C1 = 1.0 - 2.0 ** -14      # int8 deq of an identity diagonal


def test_top2_is_best_pair_by_brute_force():
    rng = np.random.default_rng(31)
    for trial in range(300):
        l = rng.standard_normal(8).astype(np.float32)
        if trial % 5 == 0:
            l[rng.integers(8)] = l[rng.integers(8)]          # plant ties
        p = np.exp(l.astype(np.float64))
        best = max(itertools.combinations(range(8), 2), key=lambda ab: (p[ab[0]] + p[ab[1]], -ab[0], -ab[1]))
        (a, b), (ga, gb) = route_top2(l)
        assert {a, b} == set(best)
        assert p[a] >= p[b]
        assert math.isclose(ga, 1.0 / (1.0 + math.exp(float(l[b]) - float(l[a]))), rel_tol=1e-14)
        assert math.isclose(ga + gb, 1.0, rel_tol=1e-15)


def test_equal_logits_pick_lowest_indices_with_half_gates():
    (a, b), (ga, gb) = route_top2(np.zeros(8, np.float32))
    assert (a, b) == (0, 1) and ga == 0.5 and gb == 0.5
    l = np.array([0, 3, 1, 3, 3, 2, 0, 0], np.float32)
    (a, b), _ = route_top2(l)
    assert (a, b) == (1, 3)


def _identity_experts(e, d, f, w1_scale=1.0):
    w13 = np.zeros((e, 2 * f, d), np.float32)
    for i in range(e):
        w13[i, :f] = np.eye(f, d) * w1_scale
        w13[i, f:] = np.eye(f, d)
    w2 = np.stack([np.eye(d, f, dtype=np.float32)] * e)
    q13, s13 = zip(*[quantize_int8(m) for m in w13])
    q2, s2 = zip(*[quantize_int8(m) for m in w2])
    return np.stack(q13), np.stack(s13), np.stack(q2), np.stack(s2)


def test_identity_experts_closed_form():
    d = f = 32
    q13, s13, q2, s2 = _identity_experts(8, d, f)
    rng = np.random.default_rng(32)
    x = round_f32_to_bf16(rng.standard_normal(d).astype(np.float32))
    xv = bf16_to_f64(x)
    logits = rng.standard_normal(8).astype(np.float32)
    y, _, _ = moe_top2(x, logits, q13, s13, q2, s2)
    want = C1 * silu(C1 * xv) * (C1 * xv)
    assert np.allclose(y, want, rtol=1e-14, atol=1e-300)


def test_silu_on_first_half_not_second():
    d = f = 32
    q13, s13, q2, s2 = _identity_experts(8, d, f, w1_scale=0.5)   # W1 = I/2, W3 = I
    x = round_f32_to_bf16(np.linspace(-3, 3, d).astype(np.float32))
    xv = bf16_to_f64(x)
    y, _, _ = moe_top2(x, np.zeros(8, np.float32), q13, s13, q2, s2)
    c_half = float(bf16_to_f64(s13[0, 0])) * 127          # deq of 0.5 on the diagonal
    want = C1 * silu(c_half * xv) * (C1 * xv)
    assert np.allclose(y, want, rtol=1e-14, atol=1e-300)
    wrong = C1 * silu(C1 * xv) * (c_half * xv)
    assert not np.allclose(y, wrong, rtol=1e-6)


def test_identical_experts_gates_sum_to_one():
    rng = np.random.default_rng(33)
    d, f = 64, 48
    w13 = (rng.standard_normal((2 * f, d)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((d, f)) * 0.02).astype(np.float32)
    q13, s13 = quantize_int8(w13)
    q2, s2 = quantize_int8(w2)
    Q13, S13 = np.stack([q13] * 8), np.stack([s13] * 8)
    Q2, S2 = np.stack([q2] * 8), np.stack([s2] * 8)
    x = round_f32_to_bf16(rng.standard_normal(d).astype(np.float32))
    for _ in range(5):
        y, _, _ = moe_top2(x, rng.standard_normal(8).astype(np.float32), Q13, S13, Q2, S2)
        y0, _, _ = moe_top2(x, np.zeros(8, np.float32), Q13, S13, Q2, S2)
        assert np.allclose(y, y0, rtol=1e-13, atol=1e-15)


def test_only_selected_experts_matter():
    rng = np.random.default_rng(34)
    d, f, e = 32, 32, 8
    w13 = (rng.standard_normal((e, 2 * f, d)) * 0.02).astype(np.float32)
    w2 = (rng.standard_normal((e, d, f)) * 0.02).astype(np.float32)
    q13, s13 = map(np.stack, zip(*[quantize_int8(m) for m in w13]))
    q2, s2 = map(np.stack, zip(*[quantize_int8(m) for m in w2]))
    x = round_f32_to_bf16(rng.standard_normal(d).astype(np.float32))
    logits = rng.standard_normal(8).astype(np.float32)
    y, (a, b), (ga, gb) = moe_top2(x, logits, q13, s13, q2, s2)
    q13b, q2b = q13.copy(), q2.copy()
    for i in range(e):
        if i not in (a, b):
            q13b[i] = 127
            q2b[i] = -127
    y2, sel2, _ = moe_top2(x, logits, q13b, s13, q2b, s2)
    assert sel2 == (a, b) and np.array_equal(y, y2)
    # and the combination is linear in the two expert outputs
    from oracle.moe import expert_ffn
    ya = expert_ffn(x, q13[a], s13[a], q2[a], s2[a])
    yb = expert_ffn(x, q13[b], s13[b], q2[b], s2[b])
    assert np.allclose(y, ga * ya + gb * yb, rtol=1e-14, atol=1e-18)


def test_silu_properties():
    # silu(0) = 0; silu(ln 3) = (3/4) ln 3 since sigmoid(ln 3) = 3/4;
    # silu(-t) = silu(t) - t; silu(t) -> t for large t and -> 0 for very negative t
    assert silu(0.0) == 0.0
    assert math.isclose(float(silu(math.log(3.0))), 0.75 * math.log(3.0), rel_tol=1e-15)
    for t in (0.3, 1.7, 5.0):
        assert math.isclose(float(silu(-t)), float(silu(t)) - t, rel_tol=1e-13)
    assert math.isclose(float(silu(40.0)), 40.0, rel_tol=1e-15)
    assert abs(float(silu(-40.0))) < 1e-15
