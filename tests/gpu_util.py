"""Helpers for GPU parity tests: device upload/download and the error metric.

The comparison metric is the max-norm relative error of an output vector,
max_i |y_gpu[i] - y_ref[i]| / max_i |y_ref[i]| (per token row for
multi-token outputs).  Elementwise relative error is ill-posed for outputs
near zero; the max-norm form is the one the tolerances are stated in:
fp32 outputs within 2e-3, bf16 outputs within 1e-2.
"""

import numpy as np

TOL_F32 = 2e-3
TOL_BF16 = 1e-2


def torch_mod():
    import torch
    return torch


def dev(a, dtype=None):
    """numpy array -> contiguous CUDA tensor (bit-preserving for uint16/uint8)."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).to("cuda")
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32)).to("cuda")
    else:
        t = torch.from_numpy(a).to("cuda")
    return t


def host_u16(t):
    return t.detach().cpu().numpy().view(np.uint16)


def host(t):
    return t.detach().cpu().numpy()


def empty(shape, dtype):
    torch = torch_mod()
    return torch.empty(shape, dtype=dtype, device="cuda")


def guarded(n, dtype, fill):
    """Output buffer with 64 guard elements on each side; returns (buf, view)."""
    torch = torch_mod()
    buf = torch.full((n + 128,), fill, dtype=dtype, device="cuda")
    return buf, buf[64:64 + n]


def bf16_bits_to_f64(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rel_err(y, ref):
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    den = np.max(np.abs(ref), axis=-1)
    num = np.max(np.abs(y - ref), axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den))


def say(*a):
    print(*a, flush=True)


def assert_same(got, want, what="repeat run"):
    """Bitwise equality, naming the differing positions when it fails."""
    got = np.asarray(got)
    want = np.asarray(want)
    if not np.array_equal(got, want):
        idx = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
        pairs = [(int(i), float(got.reshape(-1)[i]), float(want.reshape(-1)[i])) for i in idx[:8]]
        raise AssertionError(f"{what}: {idx.size} of {got.size} values differ, first (index, got, want): {pairs}")
