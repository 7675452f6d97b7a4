"""Full-size parity in the launch configuration bench.py times.

Each workload is built exactly as the bench builds it (device-generated
weights, quantized by the library, one persistent launch per decode step for
the linear sets), run once, and checked against the oracle on sampled rows:
the sampled rows' fp32 weights are regenerated from the same seeded device
generator, quantized by the ORACLE (codes and scales must match the device's
bit for bit) and multiplied in fp64; the device outputs at those rows must be
within the bf16 tolerance (the bench stores bf16 outputs) and, on a second
run with fp32 outputs, within the fp32 tolerance.  Every distinct matrix
shape of each workload is sampled (layer 0, the last layer, lm_head).
"""

import numpy as np
import pytest

from gpu_util import host, host_u16, rel_err, bf16_bits_to_f64, TOL_F32, TOL_BF16, say
from oracle.bf16 import round_f32_to_bf16, bf16_to_f64
from oracle.quant import quantize_int8, quantize_int4
from oracle.matvec import gemv_bf16, gemv_int8, gemv_int4g32, gemm_small_m

pytestmark = pytest.mark.gpu
SAMPLE = 48


def _rows(n, seed):
    rng = np.random.default_rng(seed)
    r = set(rng.choice(n, min(n, SAMPLE - 2), replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(r))


def _check_matrix(wl, q, mat, gen_w, layer_tag):
    import torch
    rows = _rows(q.n, mat.layer * 7 + mat.mid)
    w = gen_w(q.n, q.k, mat)
    ridx = torch.as_tensor(rows, device="cuda")
    w_rows = host(w.index_select(0, ridx))
    del w
    x = host_u16(q.x.view(torch.int16)).reshape(q.m, q.k) if q.m > 1 else host_u16(q.x.view(torch.int16))
    if wl.fmt == "bf16":
        wb = round_f32_to_bf16(w_rows)
        assert np.array_equal(host_u16(q.w.index_select(0, ridx)), wb)
        ref = gemv_bf16(x, wb)
    elif wl.fmt == "int8":
        qq, ss = quantize_int8(w_rows)
        assert np.array_equal(host(q.w.index_select(0, ridx)), qq), "int8 codes differ"
        assert np.array_equal(host_u16(q.aux.index_select(0, ridx)), ss), "int8 scales differ"
        ref = gemv_int8(x, qq, ss)     # x [m, k] for m token rows
    else:
        from weight_only_quantized_wq_amd.layerset import int4_group
        pp, sz = quantize_int4(w_rows, int4_group(wl.fmt, q.k))
        assert np.array_equal(host(q.w.index_select(0, ridx)), pp), "int4 codes differ"
        assert np.array_equal(host_u16(q.aux.index_select(0, ridx)), sz), "int4 scale/zero differ"
        ref = gemm_small_m(x, pp, sz) if q.m > 1 else gemv_int4g32(x, pp, sz)
    ref = ref.reshape(q.m, len(rows))
    g16 = bf16_bits_to_f64(host_u16(q.y16)).reshape(q.m, q.n)[:, rows]
    g32 = host(q.y32).reshape(q.m, q.n)[:, rows]
    e16, e32 = rel_err(g16, ref), rel_err(g32, ref)
    say(f"  {layer_tag} {mat.name} [{q.n}x{q.k}] m={q.m}: err f32={e32:.2e} bf16={e16:.2e}")
    assert e16 <= TOL_BF16 and e32 <= TOL_F32


LINEAR_SETS = ["llama2-7b-int4", "llama2-7b-int8", "llama2-7b-bf16", "llama3.1-8b-int8", "llama3.1-8b-bf16",
               "llama3.1-70b-int4-m5", "llama3.1-70b-int8-m5", "llama3.1-70b-int8", "llama2-70b-int8",
               "llama2-70b-int4", "llama2-7b-int4g128", "llama2-7b-int4pc", "int8-4096"] + \
              [f"{b}-tp{p}" for b in ("llama2-7b-int4", "llama2-7b-int8", "llama3.1-70b-int4-m5") for p in (2, 4, 8)]


@pytest.mark.parametrize("name", LINEAR_SETS)
def test_workload_full_size_sampled(name):
    import torch
    from synth.workloads import WORKLOADS, gen_w_device, gen_x_device
    from weight_only_quantized_wq_amd.layerset import LayerSet
    wl = WORKLOADS[name]
    say(f"workload {name}")
    ls = LayerSet(wl.matrices(), wl.fmt, gen_w_device(wl), gen_x_device(wl), m=wl.m)
    ls.prepare_fused(with_f32=True)
    ls.step_fused()
    torch.cuda.synchronize()
    mats = wl.matrices()
    gen_w = gen_w_device(wl)
    check = {0} if wl.model is None else {0, wl.model.layers - 1, wl.model.layers}   # first, last, lm_head
    for q, mat in zip(ls.mats, mats):
        if mat.layer in check:
            _check_matrix(wl, q, mat, gen_w, f"layer {mat.layer}")
        if wl.model is None:
            break
    del ls
    torch.cuda.empty_cache()


@pytest.mark.parametrize("launch", ["fused", "per-layer"])
def test_mixtral_full_size_sampled(launch):
    """Mixtral-8x7B MoE layers as the bench builds them (two layers; the bench
    runs 32): the selected experts' fp32 weights are regenerated and quantized
    by the oracle, whose codes must match the device's bit for bit, then the
    oracle's MoE output is compared with the device output of each layer --
    through the two-launch step (the bench's launch configuration) and
    through the single-layer call."""
    import torch
    from synth.workloads import WORKLOADS, expert_key, logits_key, moe_x_key
    from synth.gen import device_normal, device_bf16_normal
    from weight_only_quantized_wq_amd.layerset import MoELayerSet
    from oracle.moe import moe_top2
    wl = WORKLOADS["mixtral-int8"]
    mm = wl.model

    def gw(rows, cols, key):
        return device_normal((rows, cols), wl.sigma, "cuda", *expert_key(wl, key[0], key[1], key[2]))
    ls = MoELayerSet(mm.dim, mm.ffn, mm.experts, 2, gw,
                     lambda d, l: device_bf16_normal((d,), "cuda", *moe_x_key(wl, l)),
                     lambda e, l: device_normal((e,), 1.0, "cuda", *logits_key(wl, l)))
    if launch == "fused":
        ls.prepare_fused(with_f32=True, with_sel=True)
        ls.step_fused()
    else:
        for li, L in enumerate(ls.layers):
            L["y32"] = torch.empty(mm.dim, dtype=torch.float32, device="cuda")
            L["sel"] = torch.empty(2, dtype=torch.int32, device="cuda")
            ls.launch_layer(li, y32=L["y32"], sel=L["sel"])
    torch.cuda.synchronize()
    for li, L in enumerate(ls.layers):
        a, b = host(L["sel"]).tolist()
        Q13 = np.zeros((8, 2 * mm.ffn, mm.dim), np.int8)
        Q2 = np.zeros((8, mm.dim, mm.ffn), np.int8)
        S13 = np.zeros((8, 2 * mm.ffn), np.uint16)
        S2 = np.zeros((8, mm.dim), np.uint16)
        for e in (a, b):
            q13, s13 = quantize_int8(host(gw(2 * mm.ffn, mm.dim, (li, e, 0))))
            q2, s2 = quantize_int8(host(gw(mm.dim, mm.ffn, (li, e, 1))))
            assert np.array_equal(host(L["w13"][e]), q13) and np.array_equal(host_u16(L["s13"][e]), s13)
            assert np.array_equal(host(L["w2"][e]), q2) and np.array_equal(host_u16(L["s2"][e]), s2)
            Q13[e], S13[e], Q2[e], S2[e] = q13, s13, q2, s2
        x = host_u16(L["x"].view(torch.int16))
        logits = host(L["logits"])
        ref, sel_ref, _ = moe_top2(x, logits, Q13, S13, Q2, S2)
        assert tuple(sel_ref) == (a, b)
        e32 = rel_err(host(L["y32"]), ref)
        e16 = rel_err(bf16_bits_to_f64(host_u16(L["y16"])), ref)
        say(f"  mixtral {launch} layer {li} experts {(a, b)}: err f32={e32:.2e} bf16={e16:.2e}")
        assert e32 <= TOL_F32 and e16 <= TOL_BF16
