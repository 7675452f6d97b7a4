"""GPU top-2 MoE decode step vs the oracle.

Small and ragged shapes with oracle-quantized experts, the full Mixtral-8x7B
expert shape (dim 4096, ffn 14336, 8 experts) with seeded random int8 codes
and bf16 row scales, routing ties, identical experts, and the check that the
unselected experts' weights are never read (they hold codes that would change
the result).
"""

import numpy as np
import pytest

from gpu_util import dev, host, host_u16, rel_err, bf16_bits_to_f64, TOL_F32, TOL_BF16, say
from oracle.bf16 import round_f32_to_bf16
from oracle.quant import quantize_int8
from oracle.moe import moe_top2, route_top2
from synth.gen import host_normal, host_bf16_normal, host_logits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_wq_amd as m
    return m


def _experts(e, dim, f, seed):
    q13, s13, q2, s2 = [], [], [], []
    for i in range(e):
        a, b = quantize_int8(host_normal((2 * f, dim), 0.02, 960, seed, i, 0))
        c, d = quantize_int8(host_normal((dim, f), 0.02, 960, seed, i, 1))
        q13.append(a), s13.append(b), q2.append(c), s2.append(d)
    return np.stack(q13), np.stack(s13), np.stack(q2), np.stack(s2)


def _run(wq, x, logits, q13, s13, q2, s2, dim, f):
    import torch
    work = torch.empty(2 * f, dtype=torch.float32, device="cuda")
    y32 = torch.empty(dim, dtype=torch.float32, device="cuda")
    y16 = torch.empty(dim, dtype=torch.int16, device="cuda")
    sel = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    gates = torch.zeros(2, dtype=torch.float32, device="cuda")
    wq.moe_top2_gemv(dev(x), dev(logits), 8, dev(q13), dev(s13), dev(q2), dev(s2), dim, f, work, y32, y16,
                     sel, gates)
    return host(y32), host_u16(y16), tuple(host(sel).tolist()), host(gates)


def _check(got32, got16, ref):
    e32 = rel_err(got32, ref)
    e16 = rel_err(bf16_bits_to_f64(got16), ref)
    assert e32 <= TOL_F32, e32
    assert e16 <= TOL_BF16, e16
    assert np.array_equal(got16, round_f32_to_bf16(got32))
    return e32, e16


@pytest.mark.parametrize("dim,f,seed", [(64, 128, 0), (1024, 2816, 1), (4096, 512, 2), (48, 4096, 3)])
def test_moe_oracle_quantized(wq, dim, f, seed):
    say(f"moe dim={dim} f={f}")
    q13, s13, q2, s2 = _experts(8, dim, f, seed)
    x = host_bf16_normal((dim,), 961, seed, 0, 1)
    logits = host_logits(8, 961, seed, 0, 2)
    ref, sel_ref, g_ref = moe_top2(x, logits, q13, s13, q2, s2)
    y32, y16, sel, gates = _run(wq, x, logits, q13, s13, q2, s2, dim, f)
    assert sel == tuple(sel_ref)
    assert np.allclose(gates, g_ref, rtol=2e-6, atol=0)
    e = _check(y32, y16, ref)
    say(f"  sel={sel} err f32={e[0]:.2e} bf16={e[1]:.2e}")


def test_moe_ties_and_identical_experts(wq):
    dim, f = 64, 96
    q13, s13, q2, s2 = _experts(1, dim, f, 7)
    Q13, S13 = np.repeat(q13, 8, 0), np.repeat(s13, 8, 0)
    Q2, S2 = np.repeat(q2, 8, 0), np.repeat(s2, 8, 0)
    x = host_bf16_normal((dim,), 962, 0, 0, 1)
    y0, _, sel0, g0 = _run(wq, x, np.zeros(8, np.float32), Q13, S13, Q2, S2, dim, f)
    assert sel0 == (0, 1) and np.all(g0 == 0.5)
    logits = np.array([0.5, 2.0, -1.0, 2.0, 2.0, 0.0, 1.0, 1.5], np.float32)
    y1, _, sel1, _ = _run(wq, x, logits, Q13, S13, Q2, S2, dim, f)
    assert sel1 == (1, 3)
    ref, _, _ = moe_top2(x, logits, Q13, S13, Q2, S2)
    _check(y1, round_f32_to_bf16(y1), ref)
    assert rel_err(y1, y0) <= 1e-5


def test_moe_full_mixtral_shape_unselected_not_read(wq):
    import torch
    dim, f, e = 4096, 14336, 8
    say("moe full mixtral shape")
    g = torch.Generator(device="cuda")
    g.manual_seed(963)
    q13 = torch.randint(-127, 128, (e, 2 * f, dim), generator=g, device="cuda", dtype=torch.int32).to(torch.int8)
    q2 = torch.randint(-127, 128, (e, dim, f), generator=g, device="cuda", dtype=torch.int32).to(torch.int8)
    s13 = (torch.rand((e, 2 * f), generator=g, device="cuda") + 0.5) * 1.5e-4
    s2 = (torch.rand((e, dim), generator=g, device="cuda") + 0.5) * 1.5e-4
    s13b = s13.to(torch.bfloat16).view(torch.int16).contiguous()
    s2b = s2.to(torch.bfloat16).view(torch.int16).contiguous()
    x = host_bf16_normal((dim,), 963, 0, 0, 1)
    logits = host_logits(8, 963, 0, 0, 2)
    (a, b), _ = route_top2(logits)
    # unselected experts: codes that would change y if read
    for i in range(e):
        if i not in (a, b):
            q13[i].fill_(127)
            q2[i].fill_(-127)
    work = torch.empty(2 * f, dtype=torch.float32, device="cuda")
    y32 = torch.empty(dim, dtype=torch.float32, device="cuda")
    sel = torch.full((2,), -1, dtype=torch.int32, device="cuda")
    wq.moe_top2_gemv(dev(x), dev(logits), e, q13, s13b, q2, s2b, dim, f, work, y32, None, sel, None)
    got = host(y32)
    assert tuple(host(sel).tolist()) == (a, b)
    # oracle on the two selected experts only (the others are zero-filled on the host)
    Q13 = np.zeros((e, 2 * f, dim), np.int8)
    Q2 = np.zeros((e, dim, f), np.int8)
    S13 = host_u16(s13b)
    S2 = host_u16(s2b)
    for i in (a, b):
        Q13[i] = host(q13[i])
        Q2[i] = host(q2[i])
    ref, sel_ref, _ = moe_top2(x, logits, Q13, S13, Q2, S2)
    assert tuple(sel_ref) == (a, b)
    e32 = rel_err(got, ref)
    say(f"  sel={(a, b)} err f32={e32:.2e}")
    assert e32 <= TOL_F32
    # deterministic
    y2 = torch.empty(dim, dtype=torch.float32, device="cuda")
    wq.moe_top2_gemv(dev(x), dev(logits), e, q13, s13b, q2, s2b, dim, f, work, y2, None, None, None)
    assert np.array_equal(host(y2), got)


def test_moe_argument_errors(wq):
    import torch
    # raw device addresses: the binding passes them through unchecked, so
    # the library's own host checks decide
    keep = torch.zeros(4096, dtype=torch.int32, device="cuda")
    buf = keep.data_ptr()
    y = torch.zeros(64, dtype=torch.float32, device="cuda").data_ptr()
    with pytest.raises(wq.WQError) as ei:
        wq.moe_top2_gemv(buf, buf, 4, buf, buf, buf, buf, 64, 64, buf, y)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.moe_top2_gemv(buf + 2, buf, 8, buf, buf, buf, buf, 64, 64, buf, y)
    assert ei.value.status == 3
    with pytest.raises(wq.WQError) as ei:
        wq.moe_top2_gemv(buf, buf, 8, buf, buf, buf, buf, 64, 40, buf, y)
    assert ei.value.status == 2


def _step_layers(specs, dim, f):
    """Host inputs for several MoE layers: (x, logits, q13, s13, q2, s2, reference, sel, gates)."""
    out = []
    for li, seed in enumerate(specs):
        q13, s13, q2, s2 = _experts(8, dim, f, seed)
        x = host_bf16_normal((dim,), 964, seed, li, 1)
        logits = host_logits(8, 964, seed, li, 2)
        ref, sel_ref, g_ref = moe_top2(x, logits, q13, s13, q2, s2)
        out.append((x, logits, q13, s13, q2, s2, ref, tuple(sel_ref), g_ref))
    return out


@pytest.mark.parametrize("dim,f,seeds", [(64, 128, (10, 11, 12)), (1024, 2816, (13, 14)), (48, 4096, (15,)),
                                         (4096, 512, (16, 17))])
def test_moe_step_matches_oracle_and_single_layer_calls(wq, dim, f, seeds):
    """All layers as two persistent launches: every layer's routing, gates and
    output match the oracle, the single-layer call agrees, runs are bitwise
    reproducible, also replayed from a captured graph."""
    import torch
    say(f"moe step dim={dim} f={f} layers={len(seeds)}")
    hl = _step_layers(seeds, dim, f)
    bufs = []
    for (x, logits, q13, s13, q2, s2, _, _, _) in hl:
        bufs.append(dict(x=dev(x), logits=dev(logits), w13=dev(q13), s13=dev(s13), w2=dev(q2), s2=dev(s2),
                         work=torch.empty(2 * f, dtype=torch.float32, device="cuda"),
                         y32=torch.full((dim,), -7.0, dtype=torch.float32, device="cuda"),
                         y16=torch.full((dim,), 0x7BAD, dtype=torch.int16, device="cuda"),
                         sel=torch.full((2,), -1, dtype=torch.int32, device="cuda"),
                         gates=torch.zeros(2, dtype=torch.float32, device="cuda")))
    layers = [(b["x"], b["logits"], b["w13"], b["s13"], b["w2"], b["s2"], b["work"], b["y32"], b["y16"], b["sel"],
               b["gates"]) for b in bufs]
    ws = torch.empty(max(16, wq.wq_moe_step_workspace_bytes(len(layers))), dtype=torch.uint8, device="cuda")
    plan = wq.wq_moe_step_prepare(8, dim, f, layers, ws)
    wq.wq_moe_step_run(plan)
    torch.cuda.synchronize()
    first = []
    for li, (b, h) in enumerate(zip(bufs, hl)):
        x, logits, q13, s13, q2, s2, ref, sel_ref, g_ref = h
        assert tuple(host(b["sel"]).tolist()) == sel_ref
        assert np.allclose(host(b["gates"]), g_ref, rtol=2e-6, atol=0)
        e = _check(host(b["y32"]), host_u16(b["y16"]), ref)
        y1, _, _, _ = _run(wq, x, logits, q13, s13, q2, s2, dim, f)
        assert rel_err(host(b["y32"]), y1) <= 1e-5
        say(f"  layer {li} sel={sel_ref} err f32={e[0]:.2e} bf16={e[1]:.2e}")
        first.append(host(b["y32"]).copy())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        wq.wq_moe_step_run(plan)
    for rep in range(3):
        for b in bufs:
            b["y32"].fill_(-7.0)
        torch.cuda.synchronize()
        if rep == 0:
            wq.wq_moe_step_run(plan)
        else:
            g.replay()
        torch.cuda.synchronize()
        for b, f0 in zip(bufs, first):
            assert np.array_equal(host(b["y32"]), f0), f"run {rep} differs"


# The two launches' balance states sit at the end of a MoE step workspace,
# W13 then W2, each: int32 done, epoch, pad[2]; float w[8192]; float
# cost[2][8192], time[2][8192] and double cum[2][8193] by launch parity.
_MAXG = 8192
_BAL = 16 + 4 * _MAXG + 16 * _MAXG + 16 * (_MAXG + 1)


def test_moe_step_balance_feedback_runs(wq):
    """After several runs of a three-layer plan each launch's balance state
    is consistent: `done` back at zero and every launch counted, workgroup
    weights of mean 1 within their clamp's range, a positive report from
    every workgroup in both buffers, and the next launch's shares running
    from 0 to 1 in steps of w / G."""
    import torch
    dim, f = 1024, 2816
    say("moe step balance feedback")
    hl = _step_layers((21, 22, 23), dim, f)
    layers = []
    for (x, logits, q13, s13, q2, s2, _, _, _) in hl:
        layers.append((dev(x), dev(logits), dev(q13), dev(s13), dev(q2), dev(s2),
                       torch.empty(2 * f, dtype=torch.float32, device="cuda"),
                       torch.empty(dim, dtype=torch.float32, device="cuda"), None, None, None))
    nbytes = wq.wq_moe_step_workspace_bytes(len(layers))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    plan = wq.wq_moe_step_prepare(8, dim, f, layers, ws)
    for _ in range(9):
        wq.wq_moe_step_run(plan)
    torch.cuda.synchronize()
    tail = ws[nbytes - 2 * _BAL:].cpu().numpy()
    for which, (sb, G) in enumerate(((tail[:_BAL], plan.grid13), (tail[_BAL:], plan.grid2))):
        done, epoch = (int(v) for v in np.frombuffer(sb[:8].tobytes(), dtype=np.int32))
        assert done == 0 and epoch == 9, (which, done, epoch)
        o = 16
        w = np.frombuffer(sb[o:o + 4 * G].tobytes(), dtype=np.float32)
        o += 4 * _MAXG
        rep = np.frombuffer(sb[o:o + 16 * _MAXG].tobytes(), dtype=np.float32).reshape(2, 2, _MAXG)[:, :, :G]
        o += 16 * _MAXG
        cum = np.frombuffer(sb[o:o + 16 * (_MAXG + 1)].tobytes(), dtype=np.float64).reshape(2, _MAXG + 1)
        nxt = cum[epoch & 1, :G + 1]
        assert np.all((w >= 0.25) & (w <= 4.0)) and abs(float(w.mean()) - 1.0) < 1e-3, (which, w)
        assert np.all(rep > 0), which
        assert nxt[0] == 0.0 and nxt[G] == 1.0 and np.all(np.diff(nxt) > 0), which
        assert np.allclose(np.diff(nxt), w / G, rtol=1e-4, atol=1e-9), which


def test_moe_step_full_mixtral_shape_unselected_not_read(wq):
    """Two Mixtral-8x7B-shaped layers through the two-launch step, the
    unselected experts holding codes that would change the result."""
    import torch
    dim, f, e = 4096, 14336, 8
    say("moe step full mixtral shape")
    g = torch.Generator(device="cuda")
    g.manual_seed(965)
    layers, refs, bufs = [], [], []
    for li in range(2):
        q13 = torch.randint(-127, 128, (e, 2 * f, dim), generator=g, device="cuda", dtype=torch.int32).to(torch.int8)
        q2 = torch.randint(-127, 128, (e, dim, f), generator=g, device="cuda", dtype=torch.int32).to(torch.int8)
        s13 = ((torch.rand((e, 2 * f), generator=g, device="cuda") + 0.5) * 1.5e-4).to(torch.bfloat16)
        s2 = ((torch.rand((e, dim), generator=g, device="cuda") + 0.5) * 1.5e-4).to(torch.bfloat16)
        s13 = s13.view(torch.int16).contiguous()
        s2 = s2.view(torch.int16).contiguous()
        x = host_bf16_normal((dim,), 965, li, 0, 1)
        logits = host_logits(8, 965, li, 0, 2)
        (a, b), _ = route_top2(logits)
        Q13 = np.zeros((e, 2 * f, dim), np.int8)
        Q2 = np.zeros((e, dim, f), np.int8)
        for i in (a, b):
            Q13[i] = host(q13[i])
            Q2[i] = host(q2[i])
        ref, sel_ref, _ = moe_top2(x, logits, Q13, host_u16(s13), Q2, host_u16(s2))
        for i in range(e):
            if i not in (a, b):
                q13[i].fill_(127)
                q2[i].fill_(-127)
        y32 = torch.empty(dim, dtype=torch.float32, device="cuda")
        sel = torch.full((2,), -1, dtype=torch.int32, device="cuda")
        work = torch.empty(2 * f, dtype=torch.float32, device="cuda")
        bufs.append((q13, q2, s13, s2, y32, sel, work))
        layers.append((dev(x), dev(logits), q13, s13, q2, s2, work, y32, None, sel, None))
        refs.append((ref, tuple(sel_ref)))
    ws = torch.empty(max(16, wq.wq_moe_step_workspace_bytes(2)), dtype=torch.uint8, device="cuda")
    plan = wq.wq_moe_step_prepare(8, dim, f, layers, ws)
    wq.wq_moe_step_run(plan)
    torch.cuda.synchronize()
    for li, ((ref, sel_ref), b) in enumerate(zip(refs, bufs)):
        assert tuple(host(b[5]).tolist()) == sel_ref
        e32 = rel_err(host(b[4]), ref)
        say(f"  layer {li} sel={sel_ref} err f32={e32:.2e}")
        assert e32 <= TOL_F32


def test_moe_step_argument_errors(wq):
    import torch
    # raw device addresses (unchecked by the binding): the library decides
    keep = torch.zeros(4096, dtype=torch.int32, device="cuda")
    buf = keep.data_ptr()
    ykeep = torch.zeros(64, dtype=torch.float32, device="cuda")
    y = ykeep.data_ptr()
    ws = torch.empty(4096, dtype=torch.uint8, device="cuda")
    good = (buf, buf, buf, buf, buf, buf, buf, y, None, None, None)
    with pytest.raises(wq.WQError) as ei:
        wq.wq_moe_step_prepare(8, 64, 40, [good], ws)
    assert ei.value.status == 2
    with pytest.raises(wq.WQError) as ei:
        wq.wq_moe_step_prepare(8, 64, 64, [(buf + 2,) + good[1:]], ws)
    assert ei.value.status == 3
    with pytest.raises(wq.WQError) as ei:
        wq.wq_moe_step_prepare(8, 64, 64, [good] * 100, ws, 16)
    assert ei.value.status == 2
