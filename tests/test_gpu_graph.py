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
