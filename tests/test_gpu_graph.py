"""HIP graph capture of decode-step launches: every replay must reproduce the
eager result bitwise, with the program's own eager work and synchronisations
between replays (bf16, int8, int4 at several group sizes, 3- and 5-token
int4 and int8 sets, one launch per matrix, and a MoE layer)."""

import numpy as np
import pytest

from gpu_util import say, TOL_BF16
from synth.configs import Matrix
from synth.workloads import Workload, gen_w_device, gen_x_device
from synth.gen import device_normal, device_bf16_normal

pytestmark = pytest.mark.gpu


def _capture(fn):
    import torch
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("fmt,m", [("bf16", 1), ("int8", 1), ("int4g32", 1), ("int4g32", 5), ("int8", 5),
                                   ("int4g128", 1), ("int4g128", 5), ("int4pc", 3)])
def test_layerset_graph_replays_match_eager(fmt, m):
    import torch
    from weight_only_quantized_wq_amd.layerset import LayerSet
    say(f"graph replay {fmt} m={m}")
    wl = Workload("graph-test", 90, fmt, m, 0.02, None)
    mats = [Matrix("a", 0, 0, 300, 4096), Matrix("b", 0, 1, 77, 11008), Matrix("c", 1, 2, 1000, 4096)]
    ls = LayerSet(mats, fmt, gen_w_device(wl), gen_x_device(wl), m=m)
    ls.step()
    torch.cuda.synchronize()
    want = [q.y16.clone() for q in ls.mats]
    # the per-matrix calls agree with the fused step (parity-tested against
    # the oracle) to bf16 output rounding: same format, group size and token rows
    ls.prepare_fused()
    ls.step_fused()
    torch.cuda.synchronize()
    for q, w in zip(ls.mats, want):
        a = w.view(torch.bfloat16).float()
        b = q.y16.view(torch.bfloat16).float()
        assert float((a - b).abs().max() / b.abs().max()) <= TOL_BF16, f"{q.n}x{q.k}: per-matrix and fused differ"
    g = _capture(ls.step)
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        for q in ls.mats:
            q.y16.fill_(0x7BAD)                      # eager work between replays
        junk.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for q, w in zip(ls.mats, want):
            assert torch.equal(q.y16, w), f"replay {rep} differs"


def test_moe_graph_replays_match_eager():
    import torch
    from weight_only_quantized_wq_amd.layerset import MoELayerSet
    say("graph replay moe")

    def gw(rows, cols, key):
        return device_normal((rows, cols), 0.02, "cuda", 91, *key)
    ls = MoELayerSet(256, 512, 8, 2, gw, lambda d, l: device_bf16_normal((d,), "cuda", 91, l, 1),
                     lambda e, l: device_normal((e,), 1.0, "cuda", 91, l, 2))
    ls.step()
    torch.cuda.synchronize()
    want = [L["y16"].clone() for L in ls.layers]
    g = _capture(ls.step)
    for rep in range(4):
        for L in ls.layers:
            L["y16"].fill_(0x7BAD)
            L["work"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for L, w in zip(ls.layers, want):
            assert torch.equal(L["y16"], w), f"replay {rep} differs"


@pytest.mark.parametrize("fmt,m,n,k", [("int4", 5, 20000, 4096), ("int4", 2, 9000, 16384), ("int8", 5, 17000, 2048)])
def test_claiming_kernel_streams_and_graph_replays(monkeypatch, fmt, m, n, k):
    """The claiming single-matrix kernels take a claim slot per launch and
    leave it zeroed: launches alternating between two streams (which may
    overlap) and replays of a captured launch (one slot, reused) reproduce
    the eager result bitwise."""
    import torch
    import weight_only_quantized_wq_amd as wq
    monkeypatch.setenv("WQ_SMALLM_KERNEL", "claim")
    say(f"claiming kernel streams/graph {fmt} m={m} n={n} k={k}")
    if fmt == "int4":
        p = torch.randint(0, 256, (n, k // 2), dtype=torch.uint8, device="cuda")
        sz = (torch.randint(0x3A00, 0x3C00, (n, k // 32, 2), dtype=torch.int32, device="cuda")).to(torch.int16)
        call = lambda x, y: wq.wq_gemm_smallM(x, m, p, sz, n, k, y, None)
    else:
        q = torch.randint(-127, 128, (n, k), dtype=torch.int8, device="cuda")
        s = torch.randint(0x3A00, 0x3C00, (n,), dtype=torch.int32, device="cuda").to(torch.int16)
        call = lambda x, y: wq.wq_gemm_smallM_int8(x, m, q, s, n, k, y, None)
    xs = [device_bf16_normal((m, k), "cuda", 956, i, m, n, k).view(torch.int16) for i in range(2)]
    want = []
    for x in xs:
        y = torch.empty(m, n, dtype=torch.float32, device="cuda")
        call(x, y)
        torch.cuda.synchronize()
        want.append(y.clone())
    # two streams, launches alternating, each stream's output checked
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [[torch.empty(m, n, dtype=torch.float32, device="cuda") for _ in range(4)] for _ in range(2)]
    torch.cuda.synchronize()
    for r in range(4):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                call(xs[i], outs[i][r])
    torch.cuda.synchronize()
    for i in range(2):
        for r in range(4):
            assert torch.equal(outs[i][r], want[i]), f"stream {i} launch {r} differs"
    # a captured launch replayed: one slot, left zeroed by each replay
    y = torch.empty(m, n, dtype=torch.float32, device="cuda")
    g = _capture(lambda: call(xs[0], y))
    junk = torch.randn(1 << 20, device="cuda")
    for rep in range(4):
        y.fill_(-1.0)                                 # eager work between replays
        junk.mul_(1.0001).add_(0.5)
        call(xs[1], torch.empty(m, n, dtype=torch.float32, device="cuda"))   # other slots in between
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, want[0]), f"replay {rep} differs"
