"""GPU quantizers vs the oracle: codes, scales and zeros must be bit-identical.

Inputs include the hard cases of exact round-half-even: exact ties and their
1-ulp neighbours, rows/groups with subnormal scales, zero rows, constant and
one-signed tight groups (clamped codes), and ragged shapes.
"""

import numpy as np
import pytest

from gpu_util import dev, host, host_u16, empty, say
from oracle.quant import quantize_int8, quantize_int4g32, pack_int4
from synth.gen import host_normal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_wq_amd as m
    return m


def _int8_special(n_gauss, k, seed):
    w = host_normal((n_gauss, k), 0.02, 900, seed, 0, 0)
    rows = [w]
    rows.append(np.zeros((1, k), np.float32))                                 # zero row
    rows.append(host_normal((1, k), 1.0, 900, seed, 1, 0) * np.float32(1e-39))  # subnormal
    rows.append(host_normal((1, k), 1.0, 900, seed, 2, 0) * np.float32(1e30))   # huge
    s = 129.0 / 16384.0                                                        # scale of max 1.0
    ties = [(j + 0.5) * s for j in range(0, 126)]
    t = np.zeros(k, np.float32)
    t[0] = 1.0
    vals = np.array(ties + [-v for v in ties], np.float32)
    up = np.nextafter(vals, np.float32(np.inf))
    dn = np.nextafter(vals, np.float32(-np.inf))
    cat = np.concatenate([vals, up, dn])[: k - 1]
    t[1:1 + cat.size] = cat
    rows.append(t[None, :])
    return np.concatenate(rows).astype(np.float32)


@pytest.mark.parametrize("n,k", [(36, 1040), (5, 16), (1, 4), (3, 4100), (64, 4096)])
def test_quantize_int8_bitexact(wq, n, k):
    say(f"quantize_int8 n={n} k={k}")
    w = _int8_special(n, k, 1) if k >= 760 else host_normal((n, k), 0.02, 901, n, k, 0)
    q_ref, s_ref = quantize_int8(w)
    wd = dev(w)
    q = empty((w.shape[0], k), __import__("torch").int8)
    s = empty((w.shape[0],), __import__("torch").int16)
    wq.wq_quantize_int8(wd, w.shape[0], k, q, s)
    assert np.array_equal(host_u16(s), s_ref)
    assert np.array_equal(host(q), q_ref)


def _int4_special(n_gauss, k, seed):
    w = host_normal((n_gauss, k), 0.02, 910, seed, 0, 0)
    extra = np.zeros((6, k), np.float32)
    extra[0, :32] = 0.3                                      # constant, bf16 rounds away
    extra[0, 32:64] = 0.5                                    # bf16-exact constant
    s = 137.0 / 2048.0                                       # group {min 0, max 1}
    g = np.zeros(32, np.float32)
    g[1] = 1.0
    g[2:12] = [(j + 0.5) * s for j in range(10)]
    extra[1, :32] = g
    extra[1, 32:64] = g
    extra[1, 34:44] = np.nextafter(g[2:12], np.float32(np.inf))
    extra[1, 64:96] = g
    extra[1, 66:76] = np.nextafter(g[2:12], np.float32(-np.inf))
    extra[2, :32] = 1.0                                      # tight one-signed: clamps
    extra[2, 0] = np.float32(1.0) - np.float32(2.0 ** -12)
    extra[2, 1] = np.float32(1.0) + np.float32(2.0 ** -12)
    extra[3] = host_normal((k,), 1.0, 910, seed, 3, 0) * np.float32(1e-39)   # subnormal
    extra[4] = host_normal((k,), 0.02, 910, seed, 4, 0) + np.float32(0.05)   # one-signed
    extra[5, 5] = -1e-3
    return np.concatenate([w, extra]).astype(np.float32)


@pytest.mark.parametrize("n,k", [(13, 1056), (2, 32), (1, 96), (40, 4096)])
def test_quantize_int4g32_bitexact(wq, n, k):
    import torch
    say(f"quantize_int4g32 n={n} k={k}")
    w = _int4_special(n, k, 2) if k >= 96 else host_normal((n, k), 0.02, 911, n, k, 0)
    p_ref, sz_ref = quantize_int4g32(w)
    rows = w.shape[0]
    p = empty((rows, k // 2), torch.uint8)
    sz = empty((rows, k // 32, 2), torch.int16)
    wq.wq_quantize_int4g32(dev(w), rows, k, p, sz)
    assert np.array_equal(host_u16(sz), sz_ref)
    assert np.array_equal(host(p), p_ref)


def test_quantize_empty_is_noop(wq):
    import torch
    q = torch.full((4,), 7, dtype=torch.int8, device="cuda")
    s = torch.full((4,), 7, dtype=torch.int16, device="cuda")
    w = torch.zeros(16, dtype=torch.float32, device="cuda")
    wq.wq_quantize_int8(w, 0, 4, q, s)
    wq.wq_quantize_int4g32(w, 0, 32, q, s)
    torch.cuda.synchronize()
    assert host(q).tolist() == [7] * 4 and host(s).tolist() == [7] * 4


@pytest.mark.parametrize("group,n,k", [(64, 13, 1088), (128, 9, 1024), (256, 7, 2048), (64, 1, 64), (256, 40, 4096)])
def test_quantize_int4_groups_bitexact(wq, group, n, k):
    """Groups of 64/128/256 inputs: codes, scales and zeros bit-identical to
    the oracle, on the same hard cases (ties, neighbours, clamped one-signed
    groups, subnormal scales) spread over wider groups."""
    import torch
    from oracle.quant import quantize_int4
    say(f"quantize_int4 group={group} n={n} k={k}")
    w = _int4_special(n, k, 3) if k >= 96 else host_normal((n, k), 0.02, 912, n, k, 0)
    p_ref, sz_ref = quantize_int4(w, group)
    rows = w.shape[0]
    p = empty((rows, k // 2), torch.uint8)
    sz = empty((rows, k // group, 2), torch.int16)
    wq.wq_quantize_int4(dev(w), rows, k, group, p, sz)
    assert np.array_equal(host_u16(sz), sz_ref)
    assert np.array_equal(host(p), p_ref)


@pytest.mark.parametrize("n,k", [(13, 1056), (3, 32), (40, 4096), (5, 11008), (2, 28672)])
def test_quantize_int4_per_row_bitexact(wq, n, k):
    """One group per row (group == k): the wave-reduced min/max, scale, zero
    and every code bit-identical to the oracle, hard rows included."""
    import torch
    from oracle.quant import quantize_int4
    say(f"quantize_int4 per-row n={n} k={k}")
    w = _int4_special(n, k, 4) if k >= 96 else host_normal((n, k), 0.02, 913, n, k, 0)
    p_ref, sz_ref = quantize_int4(w, k)
    rows = w.shape[0]
    p = empty((rows, k // 2), torch.uint8)
    sz = empty((rows, 1, 2), torch.int16)
    wq.wq_quantize_int4(dev(w), rows, k, k, p, sz)
    assert np.array_equal(host_u16(sz), sz_ref)
    assert np.array_equal(host(p), p_ref)


@pytest.mark.parametrize("group", [32, 128, "row"])
def test_quantize_int4_zero_minimum_is_positive_zero(wq, group):
    """Groups whose minimum is zero, written as +0, -0 or both in either
    order, store z = +0 like the oracle."""
    import torch
    from oracle.quant import quantize_int4
    k = 256
    g = k if group == "row" else group
    say(f"quantize_int4 signed zeros group={group}")
    base = np.linspace(0.0, 1.0, k, dtype=np.float32)
    rows = []
    for pattern in ([0.0], [-0.0], [0.0, -0.0], [-0.0, 0.0]):
        for start in range(0, k, g):
            r = base.copy()
            r[start:start + len(pattern)] = np.array(pattern, np.float32)
            rows.append(r)
            rows.append(r[::-1].copy())
    w = np.stack(rows)
    p_ref, sz_ref = quantize_int4(w, g)
    assert np.all(sz_ref[..., 1] == 0) or g != k
    p = empty((w.shape[0], k // 2), torch.uint8)
    sz = empty((w.shape[0], k // g, 2), torch.int16)
    wq.wq_quantize_int4(dev(w), w.shape[0], k, g, p, sz)
    assert np.array_equal(host_u16(sz), sz_ref)
    assert np.array_equal(host(p), p_ref)
