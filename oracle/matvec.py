"""Dequantized decode matvec for the oracle (test infrastructure only).

At batch 1 every decode step applies each linear layer once to one token's
activation; the pages benchmark exactly that case and report the memory
bandwidth it reaches (gittoolsai "gpt-fast" README mirror, section
"基准测试", table "Tokens/Second / 内存带宽 (GB/s)").  Speculative decoding
has the larger model check several draft tokens in one pass (onegen.ai
guide, "Key Features / Speculative Decoding"), which is the same product with
a few token rows.

With W stored [N_out, K_in] as a linear layer's weight, the product is
y[m, n] = sum_k x[m, k] * deq(W)[n, k], computed here in fp64 with a BLAS
matrix product on the exactly dequantized weights.  The activation x is given
as bf16 bit patterns (or, for the MoE second projection, as fp64 values).
"""

import numpy as np

from .bf16 import bf16_to_f64
from .quant import dequantize_int8, dequantize_int4


def activations_f64(x_bits):
    """bf16 activations (bit patterns) -> fp64, exact."""
    return bf16_to_f64(x_bits)


def gemv_dequantized(x64, deq64):
    """y = x . deq^T in fp64 for x [K] or [M, K] and deq [N, K]."""
    x64 = np.asarray(x64, np.float64)
    deq64 = np.asarray(deq64, np.float64)
    if deq64.shape[1] == 0:
        return np.zeros(x64.shape[:-1] + (deq64.shape[0],), np.float64)
    return x64 @ deq64.T


def gemv_bf16(x_bits, w_bits):
    """Unquantized baseline: bf16 weights [N, K], bf16 activations."""
    return gemv_dequantized(activations_f64(x_bits), bf16_to_f64(w_bits))


def gemv_int8(x_bits, q, s):
    """int8 per-row weights: y[n] = s[n] * sum_k x[k] q[n, k]."""
    return gemv_dequantized(activations_f64(x_bits), dequantize_int8(q, s))


def gemv_int8_f64x(x64, q, s):
    """int8 per-row weights applied to fp64 activations (MoE down projection)."""
    return gemv_dequantized(x64, dequantize_int8(q, s))


def gemv_int4(x_bits, packed, sz):
    """int4 weights in groups of G = K / sz.shape[1]:
    y[n] = sum_g (s[n,g] sum_{k in g} x[k] q[n,k] + z[n,g] sum_{k in g} x[k])."""
    return gemv_dequantized(activations_f64(x_bits), dequantize_int4(packed, sz))


gemv_int4g32 = gemv_int4   # the G = 32 name


def gemm_small_m(x_bits, packed, sz):
    """Speculative verify: M token rows x [M, K] against int4 weights -> [M, N]."""
    x_bits = np.asarray(x_bits)
    if x_bits.ndim != 2:
        raise ValueError("x must be [M, K]")
    return gemv_int4g32(x_bits, packed, sz)


def gemm_small_m_int8(x_bits, q, s):
    """Speculative verify through an int8 linear: M token rows x [M, K]
    against int8 per-row weights -> [M, N], y[m, n] = s[n] sum_k x[m, k] q[n, k]."""
    x_bits = np.asarray(x_bits)
    if x_bits.ndim != 2:
        raise ValueError("x must be [M, K]")
    return gemv_int8(x_bits, q, s)
