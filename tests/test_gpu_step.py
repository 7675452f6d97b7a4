"""Whole decode step in one persistent launch (wq_decode_step_*) vs the oracle.

Each case mixes shapes that take different wave roles in the step kernel
(one wave per row, split-K across 2..7 waves, idle waves), ragged row counts
and N = 1, with oracle-quantized weights.  Every matrix's fp32 and bf16
outputs must meet the tolerances; runs are bitwise reproducible and graph
replays reproduce the eager run.
"""

import numpy as np
import pytest

from gpu_util import dev, host, host_u16, rel_err, bf16_bits_to_f64, TOL_F32, TOL_BF16, say
from oracle.bf16 import round_f32_to_bf16
from oracle.quant import quantize_int8, quantize_int4
from oracle.matvec import gemv_bf16, gemv_int8, gemv_int4g32, gemm_small_m, gemm_small_m_int8
from synth.gen import host_normal, host_bf16_normal

pytestmark = pytest.mark.gpu

SHAPES = {
    # one-token rows of one pass that share it: L lanes per row with 2 chunks
    # of each of 2 rows per lane (k = 1024, 512, 32, ...), or "wide" with up
    # to 4 (bf16: 8) chunks of one row per lane where that leaves fewer slots
    # idle (int4 k = 1376, 1536, 2752, 3072; bf16 k = 688); ragged row counts
    ("bf16", 1): [(300, 4096), (37, 11008), (5, 14336), (1, 4096), (129, 1024), (64, 8), (2, 65536), (35, 688)],
    ("int8", 1): [(300, 4096), (37, 11008), (5, 14336), (1, 4096), (129, 1024), (64, 16), (3, 28672),
                  (2, 36864), (67, 1376)],
    ("int4g32", 1): [(300, 4096), (37, 11008), (5, 14336), (1, 4096), (129, 1024), (64, 32), (3, 28672),
                     (70, 4160), (2, 73728), (67, 1376), (33, 2752), (21, 1536), (9, 3072)],
    ("int4g32", 5): [(70, 8192), (19, 28672), (1, 4096), (33, 1024), (8, 32)],
    ("int4g32", 2): [(45, 4096), (9, 16384)],
    ("int4g32", 8): [(45, 4096), (9, 16384), (3, 28672)],
    ("int4g32", 3): [(70, 8192), (19, 28672), (1, 4096), (33, 1024), (8, 32), (40, 8288)],
    ("int4g32", 4): [(45, 4096), (9, 16384), (77, 12352)],
    ("int4g32", 6): [(45, 4096), (9, 16384)],
    ("int4g32", 7): [(45, 4096), (31, 8192), (2, 32)],
    ("int4g64", 1): [(300, 4096), (37, 11008), (1, 64), (64, 28672)],
    ("int4g128", 1): [(300, 4096), (5, 14336), (129, 1024), (3, 128), (21, 1536)],
    ("int4g256", 1): [(300, 4096), (37, 11008 // 256 * 256), (1, 256), (9, 28672)],
    ("int4pc", 1): [(300, 4096), (37, 11008), (5, 14336), (1, 32), (129, 1056), (3, 28672), (13, 1376)],
    # larger int4 groups with 2..8 token rows: words per 32-input chunk of the
    # (scale, zero) window, one- and multi-window rows (k > 8192), ragged n
    ("int4g64", 2): [(45, 4096), (9, 16384), (1, 64)],
    ("int4g128", 5): [(70, 8192), (19, 28672), (33, 1024), (8, 128), (40, 8320)],
    ("int4g256", 8): [(45, 4096), (9, 16384), (3, 28672)],
    ("int4pc", 5): [(70, 8192), (19, 28672), (33, 1056), (8, 32)],
    ("int4pc", 3): [(40, 8288), (5, 96)],
    # int8 with 2..8 token rows: 16-row tiles, passes of 256 inputs (ragged
    # row counts, k not a multiple of a pass, one 16-input chunk)
    ("int8", 2): [(300, 4096), (37, 11008), (1, 16)],
    ("int8", 3): [(45, 4112), (9, 28672)],
    ("int8", 4): [(77, 8192), (33, 1040)],
    ("int8", 5): [(300, 8192), (19, 28672), (1, 4096), (33, 1024), (8, 16), (40, 8208)],
    ("int8", 6): [(45, 4096), (9, 14336)],
    ("int8", 7): [(45, 4096), (31, 8192), (2, 48)],
    ("int8", 8): [(45, 4096), (9, 16384), (3, 57344)],
}


def _build(fmt, m, seed):
    import torch
    mats, refs = [], []
    for i, (n, k) in enumerate(SHAPES[(fmt, m)]):
        w = host_normal((n, k), 0.02, 980, seed, i, 0)
        x = host_bf16_normal((m, k) if m > 1 else (k,), 980, seed, i, 1)
        if fmt == "bf16":
            wb = round_f32_to_bf16(w)
            ref = gemv_bf16(x, wb)
            W, A = dev(wb), None
        elif fmt == "int8":
            q, s = quantize_int8(w)
            ref = gemm_small_m_int8(x, q, s) if m > 1 else gemv_int8(x, q, s)
            W, A = dev(q), dev(s)
        else:
            p, sz = quantize_int4(w, k if fmt == "int4pc" else int(fmt[5:]))     # "int4g<G>" / one group per row
            ref = gemm_small_m(x, p, sz) if m > 1 else gemv_int4g32(x, p, sz)
            W, A = dev(p), dev(sz)
        y32 = torch.full((m * n,), -7.0, dtype=torch.float32, device="cuda")
        y16 = torch.full((m * n,), 0x7BAD, dtype=torch.int16, device="cuda")
        mats.append((dev(x), W, A, n, k, y32, y16))
        refs.append(ref.reshape(m, n) if m > 1 else ref.reshape(1, n))
    return mats, refs


@pytest.mark.parametrize("fmt,m", list(SHAPES))
def test_step_matches_oracle(fmt, m):
    import torch
    import weight_only_quantized_wq_amd as wq
    say(f"decode step {fmt} m={m}")
    mats, refs = _build(fmt, m, 1)
    ws = torch.empty(wq.wq_decode_step_workspace_bytes(len(mats)), dtype=torch.uint8, device="cuda")
    plan = wq.wq_decode_step_prepare(fmt, m, mats, ws)
    wq.wq_decode_step_run(plan)
    torch.cuda.synchronize()
    first = []
    for (x, W, A, n, k, y32, y16), ref in zip(mats, refs):
        g32 = host(y32).reshape(m, n)
        g16 = host_u16(y16)
        e32 = rel_err(g32, ref)
        e16 = rel_err(bf16_bits_to_f64(g16).reshape(m, n), ref)
        say(f"  n={n} k={k}: err f32={e32:.2e} bf16={e16:.2e}")
        assert e32 <= TOL_F32 and e16 <= TOL_BF16
        assert np.array_equal(g16, round_f32_to_bf16(host(y32)))
        first.append(host(y32).copy())
    # bitwise reproducible, also from a captured graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.wq_decode_step_run(plan)
    for rep in range(3):
        for mt in mats:
            mt[5].fill_(-7.0)
        torch.cuda.synchronize()
        if rep == 0:
            wq.wq_decode_step_run(plan)
        else:
            g.replay()
        torch.cuda.synchronize()
        for mt, f in zip(mats, first):
            assert np.array_equal(host(mt[5]), f), f"run {rep} differs"


def test_step_argument_errors():
    import torch
    import weight_only_quantized_wq_amd as wq
    # raw device addresses (unchecked by the binding): the library decides
    keep = torch.zeros(4096, dtype=torch.int32, device="cuda")
    buf = keep.data_ptr()
    ws = torch.empty(wq.wq_decode_step_workspace_bytes(1), dtype=torch.uint8, device="cuda")
    good = (buf, buf, buf, 4, 64, buf, None)
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g32", 9, [good], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g32", 1, [(buf, buf, buf, 4, 48, buf, None)], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g32", 1, [(buf, buf, None, 4, 64, buf, None)], ws)
    assert ei.value.status == 1
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g32", 1, [(buf + 2, buf, buf, 4, 64, buf, None)], ws)
    assert ei.value.status == 3
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g32", 1, [good], ws, 64)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g32", 1, [(buf, buf, buf, 4, 2 ** 20, buf, None)], ws)
    assert ei.value.status == 2
    # one past the longest int8 / int4 rows the single-token step kernel stages
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int8", 1, [(buf, buf, buf, 4, 36880, buf, None)], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g32", 1, [(buf, buf, buf, 4, 73760, buf, None)], ws)
    assert ei.value.status == 2
    # wider int4 groups: k a multiple of the group
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("bf16", 2, [good], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g128", 1, [(buf, buf, buf, 4, 192, buf, None)], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g256", 1, [(buf, buf, buf, 4, 73984, buf, None)], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int8", 9, [good], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int8", 5, [(buf, buf, buf, 4, 40, buf, None)], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4g64", 5, [(buf, buf, buf, 4, 2 ** 20, buf, None)], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_decode_step_prepare("int4pc", 1, [(buf, buf, buf, 4, 80, buf, None)], ws)
    assert ei.value.status == 2


@pytest.mark.parametrize("fmt,m", [("int4g32", 1), ("int8", 1), ("bf16", 1), ("int4g128", 1), ("int4pc", 1), ("int4g32", 2), ("int4g32", 5),
                                  ("int8", 5), ("int4g128", 5)])
def test_step_balance_never_changes_results(fmt, m):
    """Each launch re-cuts the workgroups' ranges from the balance state the
    previous launches measured (per-workgroup speed weights for the one-token
    and int8 kernels, XCD weights and the long-row cost factor for the int4
    verify kernel); which workgroup streams a row must never
    change the row's bits.  30 launches of one plan, and a fresh plan whose
    state starts from the prior, all give the first launch's outputs."""
    import torch
    import weight_only_quantized_wq_amd as wq
    say(f"balance {fmt} m={m}")
    mats, _ = _build(fmt, m, 2)
    ws = torch.empty(wq.wq_decode_step_workspace_bytes(len(mats)), dtype=torch.uint8, device="cuda")
    plan = wq.wq_decode_step_prepare(fmt, m, mats, ws)
    wq.wq_decode_step_run(plan)
    torch.cuda.synchronize()
    first = [(host(mt[5]).copy(), host_u16(mt[6]).copy()) for mt in mats]
    for rep in range(30):
        for mt in mats:
            mt[5].fill_(-7.0)
            mt[6].fill_(0x7BAD)
        wq.wq_decode_step_run(plan)
        torch.cuda.synchronize()
        for mt, (f32, f16) in zip(mats, first):
            assert np.array_equal(host(mt[5]), f32), f"launch {rep + 2}: fp32 outputs differ"
            assert np.array_equal(host_u16(mt[6]), f16), f"launch {rep + 2}: bf16 outputs differ"
    ws2 = torch.empty_like(ws)
    plan2 = wq.wq_decode_step_prepare(fmt, m, mats, ws2)
    for mt in mats:
        mt[5].fill_(-7.0)
    wq.wq_decode_step_run(plan2)
    torch.cuda.synchronize()
    for mt, (f32, _) in zip(mats, first):
        assert np.array_equal(host(mt[5]), f32), "a fresh plan differs"


# The balance state sits at the end of a step workspace: the per-workgroup
# state every step kernel uses (int32 done, epoch, pad[2]; float w[8192];
# float cost[2][8192], time[2][8192] and double cum[2][8193] by launch
# parity), then the verify kernel's long-row state (48 bytes: double f, t[2],
# c[2], pad).
_MAXG = 8192
_STEP_BAL, _VERIFY_BAL = 16 + 4 * _MAXG + 16 * _MAXG + 16 * (_MAXG + 1), 48


@pytest.mark.parametrize("fmt,m", [("int4g32", 1), ("int8", 5), ("int4g32", 5)])
def test_step_balance_feedback_runs(fmt, m):
    """Each launch reports into its parity's buffers, its first workgroup to
    finish turns the previous launch's reports into the shares of the launch
    after the next, and its last advances the launch count.  After a dozen
    launches: `done` back at zero and every launch counted, workgroup weights
    of mean 1 within their clamp's range, a positive report from every
    workgroup in both buffers, and the next launch's shares running from 0 to
    1 in steps of w / G; verify kernel (short and long rows in one plan): the
    long-row sums cleared and the long-row factor moved off its prior of 1.2.
    A report lost or counted twice would leave `done` non-zero."""
    import torch
    import weight_only_quantized_wq_amd as wq
    say(f"balance feedback {fmt} m={m}")
    mats, _ = _build(fmt, m, 3)
    nbytes = wq.wq_decode_step_workspace_bytes(len(mats))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    plan = wq.wq_decode_step_prepare(fmt, m, mats, ws)
    for _ in range(12):
        wq.wq_decode_step_run(plan)
    torch.cuda.synchronize()
    tail = ws[nbytes - _STEP_BAL - _VERIFY_BAL:].cpu().numpy()
    sb, vb = tail[:_STEP_BAL], tail[_STEP_BAL:]
    if fmt.startswith("int4") and m > 1:
        f, t0, t1, c0, c1 = np.frombuffer(vb[:40].tobytes(), dtype=np.float64)
        assert (t0, t1, c0, c1) == (0.0, 0.0, 0.0, 0.0)
        assert 0.5 <= f <= 4.0 and f != 1.2, f"long-row factor {f}"
    G = plan.groups
    done, epoch = (int(v) for v in np.frombuffer(sb[:8].tobytes(), dtype=np.int32))
    assert done == 0, f"{done} reports left over"
    assert epoch == 12, f"{epoch} launches counted"
    o = 16
    w = np.frombuffer(sb[o:o + 4 * G].tobytes(), dtype=np.float32)
    o += 4 * _MAXG
    rep = np.frombuffer(sb[o:o + 16 * _MAXG].tobytes(), dtype=np.float32).reshape(2, 2, _MAXG)[:, :, :G]
    o += 16 * _MAXG
    cum = np.frombuffer(sb[o:o + 16 * (_MAXG + 1)].tobytes(), dtype=np.float64).reshape(2, _MAXG + 1)
    nxt = cum[epoch & 1, :G + 1]
    # clamped to [0.5, 2], then scaled to mean 1
    assert np.all((w >= 0.25) & (w <= 4.0)) and abs(float(w.mean()) - 1.0) < 1e-3, w
    assert np.all(rep > 0), "a workgroup's report is missing"
    assert nxt[0] == 0.0 and nxt[G] == 1.0 and np.all(np.diff(nxt) > 0)
    assert np.allclose(np.diff(nxt), w / G, rtol=1e-4, atol=1e-9)
