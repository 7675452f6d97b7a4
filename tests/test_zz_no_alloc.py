"""moe_top2_gemv_noalloc (no caller workspace: the SwiGLU intermediate sits in
the library's static device scratch) against moe_top2_gemv on the same
inputs, through the C ABI.  The same kernels run on both paths, so outputs,
selections and gates must agree bit for bit.  Two calls in a row, the second
with a smaller layer, check that the shared scratch carries nothing over;
a third call at the scratch's limit (f = 16384) and the refusal of a larger
f bound the static array."""

import ctypes

import numpy as np
import pytest

from gpu_util import dev, host, host_u16, rel_err, TOL_F32, say
from oracle.quant import quantize_int8
from oracle.moe import moe_top2
from synth.gen import host_normal, host_bf16_normal, host_logits

pytestmark = pytest.mark.gpu


def _layer(dim, f, seed, oracle_q=True):
    if oracle_q:
        q13, s13, q2, s2 = [], [], [], []
        for i in range(8):
            a, b = quantize_int8(host_normal((2 * f, dim), 0.02, 990, seed, i, 0))
            c, d = quantize_int8(host_normal((dim, f), 0.02, 990, seed, i, 1))
            q13.append(a), s13.append(b), q2.append(c), s2.append(d)
        q13, s13, q2, s2 = map(np.stack, (q13, s13, q2, s2))
    else:
        rng = np.random.default_rng(seed)
        q13 = rng.integers(-127, 128, (8, 2 * f, dim), dtype=np.int8)
        q2 = rng.integers(-127, 128, (8, dim, f), dtype=np.int8)
        s13 = np.full((8, 2 * f), 0x3A80, np.uint16)   # bf16 2^-10
        s2 = np.full((8, dim), 0x3A80, np.uint16)
    x = host_bf16_normal((dim,), 991, seed, 0, 1)
    logits = host_logits(8, 991, seed, 0, 2)
    return x, logits, q13, s13, q2, s2


def _both(wq, dim, f, L):
    import torch
    x, logits, q13, s13, q2, s2 = [dev(a) for a in L]
    out = {}
    for path in ("workspace", "noalloc"):
        y32 = torch.full((dim,), float("nan"), dtype=torch.float32, device="cuda")
        y16 = torch.full((dim,), -1, dtype=torch.int16, device="cuda")
        sel = torch.full((2,), -1, dtype=torch.int32, device="cuda")
        gates = torch.full((2,), float("nan"), dtype=torch.float32, device="cuda")
        if path == "workspace":
            work = torch.empty(2 * f, dtype=torch.float32, device="cuda")
            wq.moe_top2_gemv(x, logits, 8, q13, s13, q2, s2, dim, f, work, y32, y16, sel, gates)
        else:
            wq.moe_top2_gemv_noalloc(x, logits, 8, q13, s13, q2, s2, dim, f, y32, y16, sel, gates)
        torch.cuda.synchronize()
        out[path] = (host(y32), host_u16(y16), host(sel), host(gates))
    a, b = out["workspace"], out["noalloc"]
    for u, v in zip(a, b):
        assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), "noalloc differs from moe_top2_gemv"
    return b


def test_noalloc_matches_workspace_call_twice_then_smaller(wq_lib):
    wq = wq_lib
    # first call: a larger layer; second: a smaller one in the same scratch
    for dim, f, seed in [(1024, 2816, 0), (64, 128, 1)]:
        say(f"moe noalloc dim={dim} f={f}")
        L = _layer(dim, f, seed)
        y32, y16, sel, gates = _both(wq, dim, f, L)
        ref, sel_ref, _ = moe_top2(*L)
        assert tuple(sel.tolist()) == tuple(sel_ref)
        assert rel_err(y32, ref) <= TOL_F32


def test_noalloc_at_scratch_limit_and_refuses_beyond(wq_lib):
    wq = wq_lib
    dim, f = 256, 16384
    say(f"moe noalloc at the limit dim={dim} f={f}")
    _both(wq, dim, f, _layer(dim, f, 2, oracle_q=False))
    import torch
    # beyond the scratch: refused on the host (status 2) before any access,
    # so small device buffers stand in for the experts
    z = torch.zeros(1 << 20, dtype=torch.int8, device="cuda")
    y = torch.empty(dim, dtype=torch.float32, device="cuda")
    p = z.data_ptr()
    rc = wq.lib.moe_top2_gemv_noalloc(p, p, 8, p, p, p, p, dim, 16400, y.data_ptr(), None, None, None, None)
    assert rc == 2 and "scratch" in wq.last_error()


def test_noalloc_raw_c_abi_symbol(wq_lib):
    """The symbol is called straight through ctypes (no binding wrapper)."""
    import torch
    wq = wq_lib
    dim, f = 32, 48
    x, logits, q13, s13, q2, s2 = [dev(a) for a in _layer(dim, f, 3)]
    y = torch.empty(dim, dtype=torch.float32, device="cuda")
    fn = wq.lib.moe_top2_gemv_noalloc
    rc = fn(x.data_ptr(), logits.data_ptr(), 8, q13.data_ptr(), s13.data_ptr(), q2.data_ptr(), s2.data_ptr(),
            dim, f, y.data_ptr(), None, None, None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, wq.last_error()
    torch.cuda.synchronize()
    ref, _, _ = moe_top2(*_layer(dim, f, 3))
    assert rel_err(host(y), ref) <= TOL_F32


@pytest.fixture(scope="module")
def wq_lib():
    import weight_only_quantized_wq_amd as m
    return m
