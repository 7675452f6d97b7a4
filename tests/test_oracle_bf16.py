"""Pins for the oracle's fp32 -> bf16 rounding (CPU only).

Pinned against (1) exact rational nearest-even rounding and (2) torch's CPU
bf16 conversion, a library routine independent of the oracle.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from exact import f32_of_bits, round_to_bf16, frac_of_bf16
from oracle.bf16 import round_f32_to_bf16, bf16_to_f32, bf16_to_f64


def _finite_bits_grid():
    his = np.arange(0, 1 << 16, dtype=np.uint32)
    his = his[((his >> 7) & 0xFF) != 0xFF]                 # finite exponents only
    los = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    return (his[:, None] << 16 | los[None, :]).ravel()


def test_exact_nearest_even_on_grid():
    bits = _finite_bits_grid()
    rng = np.random.default_rng(1)
    pick = rng.choice(bits.size, 12000, replace=False)
    # always include every exact tie of the positive normal range's first rows
    ties = (np.arange(0x0080, 0x0080 + 512, dtype=np.uint32) << 16) | 0x8000
    sample = np.concatenate([bits[pick], ties])
    got = round_f32_to_bf16(sample.view(np.float32))
    for b, h in zip(sample.tolist(), got.tolist()):
        v = Fraction(f32_of_bits(b))
        want = round_to_bf16(v)
        if abs(want) >= Fraction(2) ** 128:                     # rounds past the largest finite
            assert h & 0x7FFF == 0x7F80
            continue
        have = frac_of_bf16(h)
        if want == 0:
            assert have == 0
        else:
            assert have == want, hex(b)


def test_matches_torch_cpu_conversion():
    rng = np.random.default_rng(2)
    vals = np.concatenate([
        rng.standard_normal(50000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),      # subnormals
        np.clip(rng.standard_normal(20000) * 1.5e38, -3.39e38, 3.39e38).astype(np.float32),  # near overflow
        _finite_bits_grid()[::7].view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, -3.3895314e38], np.float32),
    ])
    want = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = round_f32_to_bf16(vals)
    assert np.array_equal(got, want)


def test_nan_maps_to_quiet_nan():
    out = round_f32_to_bf16(np.array([np.nan], np.float32))
    assert out[0] == 0x7FC0


def test_decode_is_exact_inverse_on_bf16_values():
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    finite = ((h.astype(np.uint32) >> 7) & 0xFF) != 0xFF
    f = bf16_to_f32(h[finite])
    assert np.array_equal(round_f32_to_bf16(f), h[finite])
    assert np.array_equal(bf16_to_f64(h[finite]), f.astype(np.float64))


@pytest.mark.parametrize("value,bits", [(1.0, 0x3F80), (-2.0, 0xC000), (1.0 / 127, 0x3C01),
                                        (1.0 / 15, 0x3D89), (0.0, 0x0000)])
def test_known_values(value, bits):
    assert round_f32_to_bf16(np.array([value], np.float32))[0] == bits
