"""GPU decode matvecs (bf16, int8, int4 G=32, small-M verify) vs the oracle.

Quantized weights come from the ORACLE's quantizers (host), so these tests
check the matvec kernels alone.  Shapes span every launch plan (one wave per
row up to 16 waves per row), several row batches and ragged tails in both N
and the per-wave chunk coverage of K; K = 0 and N = 1 are included.  fp32
outputs must be within 2e-3 and bf16 outputs within 1e-2 (max-norm relative
error against the fp64 oracle); repeated calls must be bitwise identical and
must not write outside the output.
"""

import numpy as np
import pytest

from gpu_util import (assert_same, dev, host, host_u16, guarded, rel_err, bf16_bits_to_f64, TOL_F32, TOL_BF16, say)
from oracle.bf16 import round_f32_to_bf16
from oracle.quant import quantize_int8, quantize_int4g32
from oracle.matvec import gemv_bf16, gemv_int8, gemv_int4g32, gemm_small_m
from synth.gen import host_normal, host_bf16_normal

pytestmark = pytest.mark.gpu
SENT = -12345.0


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_wq_amd as m
    return m


def _d(a):
    """Upload; an empty array becomes a small zero buffer (k = 0 still needs
    valid, aligned pointers)."""
    if a.size == 0:
        return dev(np.zeros(64, a.dtype))
    return dev(a)


def _outputs(n, m=1):
    import torch
    b32, y32 = guarded(m * n, torch.float32, SENT)
    b16, y16 = guarded(m * n, torch.int16, 0x7BAD)
    return (b32, y32), (b16, y16)


def _check_guards(b32, b16, n):
    h32 = host(b32)
    h16 = host(b16)
    assert np.all(h32[:64] == SENT) and np.all(h32[64 + n:] == SENT)
    assert np.all(h16[:64] == 0x7BAD) and np.all(h16[64 + n:] == 0x7BAD)


def _compare(y32, y16, ref, shape):
    got32 = host(y32).reshape(shape)
    got16 = bf16_bits_to_f64(host_u16(y16)).reshape(shape)
    e32 = rel_err(got32, ref)
    e16 = rel_err(got16, ref)
    assert e32 <= TOL_F32, e32
    assert e16 <= TOL_BF16, e16
    # the bf16 output is the fp32 output rounded to nearest-even
    assert np.array_equal(host_u16(y16), round_f32_to_bf16(host(y32)))
    return e32, e16


BF16_SHAPES = [(37, 8), (5, 1024), (300, 4096), (129, 3584), (40, 11008), (33, 14336), (9, 28672),
               (3, 65536), (1, 4096), (7, 0)]


@pytest.mark.parametrize("n,k", BF16_SHAPES)
def test_gemv_bf16(wq, n, k):
    say(f"gemv_bf16 n={n} k={k}")
    w = round_f32_to_bf16(host_normal((n, k), 0.02, 920, n, k, 0))
    x = host_bf16_normal((k,), 920, n, k, 1)
    ref = gemv_bf16(x, w)
    (b32, y32), (b16, y16) = _outputs(n)
    wd, xd = _d(w), _d(x)
    wq.wq_gemv_bf16(xd, wd, n, k, y32, y16)
    e = _compare(y32, y16, ref, (n,))
    _check_guards(b32, b16, n)
    first = host(y32).copy()
    wq.wq_gemv_bf16(xd, wd, n, k, y32, y16)
    assert_same(host(y32), first)
    say(f"  err f32={e[0]:.2e} bf16={e[1]:.2e}")


INT8_SHAPES = [(37, 16), (5, 1024), (300, 4096), (129, 4112), (40, 11008), (33, 14336), (9, 28672),
               (3, 65536), (1, 4096), (7, 0)]


@pytest.mark.parametrize("n,k", INT8_SHAPES)
def test_gemv_int8(wq, n, k):
    say(f"gemv_int8 n={n} k={k}")
    w = host_normal((n, k), 0.02, 930, n, k, 0)
    q, s = quantize_int8(w)
    x = host_bf16_normal((k,), 930, n, k, 1)
    ref = gemv_int8(x, q, s)
    (b32, y32), (b16, y16) = _outputs(n)
    qd, sd, xd = _d(q), _d(s), _d(x)
    wq.wq_gemv_int8(xd, qd, sd, n, k, y32, y16)
    e = _compare(y32, y16, ref, (n,))
    _check_guards(b32, b16, n)
    first = host(y32).copy()
    wq.wq_gemv_int8(xd, qd, sd, n, k, y32, None)
    assert_same(host(y32), first)
    say(f"  err f32={e[0]:.2e} bf16={e[1]:.2e}")


INT4_SHAPES = [(37, 32), (5, 1024), (300, 4096), (129, 8192), (40, 11008), (33, 14336), (17, 28672),
               (9, 57344), (2, 131072), (1, 4096), (7, 0)]


@pytest.mark.parametrize("n,k", INT4_SHAPES)
def test_gemv_int4g32(wq, n, k):
    say(f"gemv_int4g32 n={n} k={k}")
    w = host_normal((n, k), 0.02, 940, n, k, 0)
    p, sz = quantize_int4g32(w) if k else (np.zeros((n, 0), np.uint8), np.zeros((n, 0, 2), np.uint16))
    x = host_bf16_normal((k,), 940, n, k, 1)
    ref = gemv_int4g32(x, p, sz)
    (b32, y32), (b16, y16) = _outputs(n)
    pd, szd, xd = _d(p), _d(sz), _d(x)
    wq.wq_gemv_int4g32(xd, pd, szd, n, k, y32, y16)
    e = _compare(y32, y16, ref, (n,))
    _check_guards(b32, b16, n)
    first = host(y32).copy()
    wq.wq_gemv_int4g32(xd, pd, szd, n, k, y32, None)
    assert_same(host(y32), first)
    say(f"  err f32={e[0]:.2e} bf16={e[1]:.2e}")


# m >= 2 runs on the matrix cores with K windows of 256 groups: the cases
# cover one window, several, a ragged last window (k = 8288, 12352, 8224),
# matrices with more row blocks than resident workgroups (3 to 8 blocks per
# workgroup with 1 to 32 items each, every token count, ragged last blocks),
# and k = 0
SMALLM_CASES = [(m, n, k) for m in range(1, 9) for (n, k) in [(45, 4096), (3, 32), (70, 8192)]] + \
    [(m, 21, 16384) for m in (2, 5, 6, 8)] + [(m, 19, 28672) for m in (2, 3, 4, 5, 7, 8)] + \
    [(5, 8, 32768), (1, 10, 131072), (5, 6, 131072), (5, 50, 8288), (7, 37, 12352), (3, 100, 8224),
    (2, 9, 0), (6, 9, 0), (5, 16411, 512), (3, 18000, 8224), (8, 17000, 4128), (2, 20000, 16416),
    (5, 31990, 1024), (6, 55999, 1024), (2, 23999, 4096), (4, 39995, 256), (3, 40000, 2048)] + \
    [(m, 49999, 256) for m in (2, 3, 4, 5, 7, 8)] + [(5, 50011, 1024), (8, 49300, 5376)]


@pytest.mark.parametrize("m,n,k", SMALLM_CASES)
def test_gemm_small_m(wq, m, n, k):
    say(f"gemm_smallM m={m} n={n} k={k}")
    w = host_normal((n, k), 0.015, 950, m, n, k)
    p, sz = quantize_int4g32(w)
    x = host_bf16_normal((m, k), 950, m, n, k + 1)
    ref = gemm_small_m(x, p, sz)
    (b32, y32), (b16, y16) = _outputs(n, m)
    pd, szd, xd = _d(p), _d(sz), _d(x)
    wq.wq_gemm_smallM(xd, m, pd, szd, n, k, y32, y16)
    e = _compare(y32, y16, ref, (m, n))
    _check_guards(b32, b16, m * n)
    # each token row matches the single-token matvec
    import torch
    one = torch.empty(n, dtype=torch.float32, device="cuda")
    got = host(y32).reshape(m, n)
    for i in range(m):
        wq.wq_gemv_int4g32(xd if k == 0 else xd[i], pd, szd, n, k, one, None)
        assert rel_err(host(one), got[i]) <= 1e-5
    say(f"  err f32={e[0]:.2e} bf16={e[1]:.2e}")


def test_n_zero_is_noop(wq):
    import torch
    y = torch.full((4,), SENT, dtype=torch.float32, device="cuda")
    x = torch.zeros(64, dtype=torch.int16, device="cuda")
    w = torch.zeros(64 * 4, dtype=torch.int16, device="cuda")
    sz = torch.zeros(16, dtype=torch.int16, device="cuda")
    wq.wq_gemv_bf16(x, w, 0, 64, y, None)
    wq.wq_gemv_int8(x, w, sz, 0, 64, y, None)
    wq.wq_gemv_int4g32(x, w, sz, 0, 64, y, None)
    wq.wq_gemm_smallM(x, 1, w, sz, 0, 64, y, None)
    torch.cuda.synchronize()
    assert np.all(host(y) == SENT)


def test_misaligned_pointers_rejected(wq):
    import torch
    x = torch.zeros(256, dtype=torch.int16, device="cuda")
    w = torch.zeros(4096, dtype=torch.int16, device="cuda")
    sz = torch.zeros(64, dtype=torch.int16, device="cuda")
    y = torch.zeros(16, dtype=torch.float32, device="cuda")
    bad = x.data_ptr() + 2
    for call in (lambda: wq.wq_gemv_bf16(bad, w, 4, 64, y, None),
                 lambda: wq.wq_gemv_int8(bad, w, sz, 4, 64, y, None),
                 lambda: wq.wq_gemv_int4g32(bad, w, sz, 4, 64, y, None),
                 lambda: wq.wq_gemm_smallM(bad, 2, w, sz, 4, 64, y, None),
                 lambda: wq.wq_gemv_int4g32(x, w, sz.data_ptr() + 2, 4, 64, y, None)):
        with pytest.raises(wq.WQError) as ei:
            call()
        assert ei.value.status == 3


GROUP_SHAPES = [(64, 37, 64), (128, 300, 4096), (256, 40, 11008 // 256 * 256), (64, 40, 11008), (128, 17, 28672),
                (256, 2, 131072), (128, 7, 0)]


@pytest.mark.parametrize("group,n,k", GROUP_SHAPES)
def test_gemv_int4_groups(wq, group, n, k):
    """int4 with groups of 64/128/256: each 32-input chunk applies its group's
    (scale, zero); the same tolerances as G = 32."""
    from oracle.quant import quantize_int4
    from oracle.matvec import gemv_int4
    say(f"gemv_int4 group={group} n={n} k={k}")
    w = host_normal((n, k), 0.02, 941, n, k, group)
    p, sz = quantize_int4(w, group) if k else (np.zeros((n, 0), np.uint8), np.zeros((n, 0, 2), np.uint16))
    x = host_bf16_normal((k,), 941, n, k, 1)
    ref = gemv_int4(x, p, sz) if k else np.zeros(n)
    (b32, y32), (b16, y16) = _outputs(n)
    pd, szd, xd = _d(p), _d(sz), _d(x)
    wq.wq_gemv_int4(xd, pd, szd, n, k, group, y32, y16)
    e = _compare(y32, y16, ref, (n,))
    _check_guards(b32, b16, n)
    say(f"  err f32={e[0]:.2e} bf16={e[1]:.2e}")


@pytest.mark.parametrize("n,k", [(37, 32), (300, 4096), (40, 11008), (17, 28672), (2, 131072), (7, 96)])
def test_gemv_int4_per_row(wq, n, k):
    """One group per row: every chunk, the padding past the row included,
    reads the row's single (scale, zero) word."""
    from oracle.quant import quantize_int4
    from oracle.matvec import gemv_int4
    say(f"gemv_int4 per-row n={n} k={k}")
    w = host_normal((n, k), 0.02, 942, n, k, 0)
    p, sz = quantize_int4(w, k)
    x = host_bf16_normal((k,), 942, n, k, 1)
    ref = gemv_int4(x, p, sz)
    (b32, y32), (b16, y16) = _outputs(n)
    wq.wq_gemv_int4(_d(x), _d(p), _d(sz), n, k, k, y32, y16)
    e = _compare(y32, y16, ref, (n,))
    _check_guards(b32, b16, n)
    say(f"  err f32={e[0]:.2e} bf16={e[1]:.2e}")


I8M_CASES = [(m, n, k) for m in range(1, 9) for (n, k) in [(45, 4096), (3, 16), (70, 8192)]] + \
    [(m, 19, 28672) for m in (2, 5, 8)] + [(5, 300, 4112), (3, 17, 57344), (8, 5, 1 << 17), (5, 7, 0),
    (5, 16411, 272), (2, 16448, 1024), (8, 20000, 528), (4, 16384, 0),
    (8, 8200, 16400), (3, 9000, 16384)]


@pytest.mark.parametrize("m,n,k", I8M_CASES)
def test_gemm_small_m_int8(wq, m, n, k):
    """m token rows through one int8 linear (16-row tiles on the matrix
    cores, passes split across a workgroup's waves) vs the oracle; each row
    matches the one-token int8 matvec."""
    import torch
    from oracle.quant import quantize_int8
    from oracle.matvec import gemm_small_m_int8
    say(f"gemm_smallM_int8 m={m} n={n} k={k}")
    w = host_normal((n, k), 0.02, 951, m, n, k)
    q, s = quantize_int8(w)
    x = host_bf16_normal((m, k), 951, m, n, k + 1)
    ref = gemm_small_m_int8(x, q, s) if k else np.zeros((m, n))
    (b32, y32), (b16, y16) = _outputs(n, m)
    qd, sd, xd = _d(q), dev(s), _d(x)
    wq.wq_gemm_smallM_int8(xd, m, qd, sd, n, k, y32, y16)
    e = _compare(y32, y16, ref, (m, n))
    _check_guards(b32, b16, m * n)
    if 0 < k <= 65536:    # the one-token int8 matvec's row limit
        one = torch.empty(n, dtype=torch.float32, device="cuda")
        got = host(y32).reshape(m, n)
        for i in range(m):
            wq.wq_gemv_int8(xd[i], qd, sd, n, k, one, None)
            assert rel_err(host(one), got[i]) <= 1e-5
    say(f"  err f32={e[0]:.2e} bf16={e[1]:.2e}")


GROUP_SMALLM_CASES = [(2, 64, 45, 4096), (3, 128, 70, 8192), (5, 128, 19, 28672), (5, 256, 33, 1024),
                      (8, 64, 21, 16384), (5, 0, 40, 8288), (4, 0, 7, 96), (6, 256, 9, 131072 // 2),
                      (5, 128, 49999, 1024), (3, 0, 50000, 512), (7, 64, 49153, 2048)]


@pytest.mark.parametrize("m,group,n,k", GROUP_SMALLM_CASES)
def test_gemm_small_m_int4_groups(wq, m, group, n, k):
    """m token rows through int4 weights with groups of 64/128/256 inputs or
    one group per row (group 0 here: group = k), vs the oracle."""
    from oracle.quant import quantize_int4
    g = group or k
    say(f"gemm_smallM_int4 m={m} group={g} n={n} k={k}")
    w = host_normal((n, k), 0.015, 952, m, n, k)
    p, sz = quantize_int4(w, g)
    x = host_bf16_normal((m, k), 952, m, n, k + 1)
    ref = gemm_small_m(x, p, sz)
    (b32, y32), (b16, y16) = _outputs(n, m)
    wq.wq_gemm_smallM_int4(dev(x), m, dev(p), dev(sz), n, k, g, y32, y16)
    e = _compare(y32, y16, ref, (m, n))
    _check_guards(b32, b16, m * n)
    say(f"  err f32={e[0]:.2e} bf16={e[1]:.2e}")


# The two matrix-core kernels for 2..5 token rows (WQ_SMALLM_KERNEL forces
# one): 1..16 (scale, zero) windows per 32-row block, one block or many more
# blocks than workgroups (blocks claimed at run time), ragged last blocks,
# every group size the claiming kernel takes.
KERNEL_CASES = [(5, 32, 45, 4096), (2, 32, 3, 32), (5, 32, 70, 8192), (3, 32, 16411, 512), (4, 32, 39995, 256),
                (5, 32, 49999, 1024), (2, 32, 9000, 16384), (3, 32, 40000, 2048), (4, 32, 9001, 8192),
                (5, 128, 20000, 4096), (2, 0, 30001, 1024), (3, 64, 12345, 8192)]


@pytest.mark.parametrize("m,group,n,k", KERNEL_CASES)
def test_gemm_small_m_kernels(wq, monkeypatch, m, group, n, k):
    """The fixed-stride and the claiming matrix-core kernels each match the
    oracle, each other to fp32 rounding, and themselves bit for bit on a
    second call (the claiming kernel's blocks go to whichever workgroup
    claims them first)."""
    from oracle.quant import quantize_int4
    g = group or k
    say(f"kernels m={m} group={g} n={n} k={k}")
    w = host_normal((n, k), 0.015, 954, m, n, k)
    p, sz = quantize_int4(w, g)
    x = host_bf16_normal((m, k), 954, m, n, k + 1)
    ref = gemm_small_m(x, p, sz)
    pd, szd, xd = _d(p), _d(sz), _d(x)
    got = {}
    for kind in ("split", "claim"):
        monkeypatch.setenv("WQ_SMALLM_KERNEL", kind)
        runs = []
        for _ in range(2):
            (b32, y32), (b16, y16) = _outputs(n, m)
            wq.wq_gemm_smallM_int4(xd, m, pd, szd, n, k, g, y32, y16)
            _compare(y32, y16, ref, (m, n))
            _check_guards(b32, b16, m * n)
            runs.append(host(y32).reshape(m, n))
        assert_same(runs[1], runs[0])
        got[kind] = runs[0]
    assert rel_err(got["split"], got["claim"]) <= 1e-5


# The int8 counterparts (WQ_SMALLM_KERNEL forces one): batches of 1, 2 and 4
# tiles, 1..32 units of 8 passes per batch, more batches than workgroups,
# ragged last batches and passes.
I8_KERNEL_CASES = [(5, 45, 4096), (2, 3, 16), (8, 70, 8192), (3, 16411, 272), (5, 16448, 1024), (8, 20000, 528),
                   (4, 9000, 16384), (2, 8200, 32768), (6, 17000, 4112), (7, 16400, 2048)]


@pytest.mark.parametrize("m,n,k", I8_KERNEL_CASES)
def test_gemm_small_m_int8_kernels(wq, monkeypatch, m, n, k):
    """The fixed-stride and the claiming int8 matrix-core kernels each match
    the oracle, each other to fp32 rounding, and themselves bit for bit."""
    from oracle.matvec import gemm_small_m_int8
    say(f"int8 kernels m={m} n={n} k={k}")
    w = host_normal((n, k), 0.02, 955, m, n, k)
    q, s = quantize_int8(w)
    x = host_bf16_normal((m, k), 955, m, n, k + 1)
    ref = gemm_small_m_int8(x, q, s)
    qd, sd, xd = _d(q), dev(s), _d(x)
    got = {}
    for kind in ("split", "claim"):
        monkeypatch.setenv("WQ_SMALLM_KERNEL", kind)
        runs = []
        for _ in range(2):
            (b32, y32), (b16, y16) = _outputs(n, m)
            wq.wq_gemm_smallM_int8(xd, m, qd, sd, n, k, y32, y16)
            _compare(y32, y16, ref, (m, n))
            _check_guards(b32, b16, m * n)
            runs.append(host(y32).reshape(m, n))
        assert_same(runs[1], runs[0])
        got[kind] = runs[0]
    assert rel_err(got["split"], got["claim"]) <= 1e-5


ENGINE_CASES = [(fmt, m, n, k) for fmt in ("int4", "int8") for m in (2, 3, 5)
                for (n, k) in [(45, 4096), (70, 8192), (3, 32), (130, 16384), (7, 0)]] + \
    [("int4", m, 19, 28672) for m in (2, 3, 5)] + [("int4", 5, 2, 32768), ("int8", 2, 9, 28672)]


@pytest.mark.parametrize("fmt,m,n,k", ENGINE_CASES)
def test_gemm_small_m_engines(wq, monkeypatch, fmt, m, n, k):
    """The vector-ALU and matrix-core kernels for 2, 3 and 5 token rows
    (WQ_SMALLM_ENGINE forces one; rows past a vector-ALU plan's reach run on
    the matrix cores) each match the oracle, and each other to fp32
    rounding."""
    from oracle.quant import quantize_int8
    from oracle.matvec import gemm_small_m_int8
    say(f"engines {fmt} m={m} n={n} k={k}")
    w = host_normal((n, k), 0.02, 953, m, n, k)
    x = host_bf16_normal((m, k), 953, m, n, k + 1)
    if fmt == "int4":
        p, sz = quantize_int4g32(w)
        ref = gemm_small_m(x, p, sz) if k else np.zeros((m, n))
        args = (_d(p), _d(sz))
    else:
        q, s = quantize_int8(w)
        ref = gemm_small_m_int8(x, q, s) if k else np.zeros((m, n))
        args = (_d(q), dev(s))
    xd = _d(x)
    got = {}
    for engine in ("valu", "mfma"):
        monkeypatch.setenv("WQ_SMALLM_ENGINE", engine)
        (b32, y32), (b16, y16) = _outputs(n, m)
        if fmt == "int4":
            wq.wq_gemm_smallM(xd, m, args[0], args[1], n, k, y32, y16)
        else:
            wq.wq_gemm_smallM_int8(xd, m, args[0], args[1], n, k, y32, y16)
        _compare(y32, y16, ref, (m, n))
        _check_guards(b32, b16, m * n)
        got[engine] = host(y32).reshape(m, n)
    assert rel_err(got["valu"], got["mfma"]) <= 1e-5
