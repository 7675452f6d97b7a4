"""Top-2 mixture-of-experts decode for the oracle (test infrastructure only).

The pages support Mixtral 8x7B, a sparse mixture of experts, and benchmark
its int8 weight-only variant on one GPU at batch 1 (gittoolsai "gpt-fast"
README mirror, section "Mixtral 8x7B", tokens/s table by GPU count).  They
state neither the routing nor the expert FFN.  Readings taken:

* Routing: softmax over the 8 router logits, keep the two largest
  probabilities (equal values: the lower expert index first), renormalise
  the two to sum to one.
* Expert FFN: SwiGLU, y_e = W2_e (silu(W1_e x) * (W3_e x)), with W1 and W3
  stacked as one [2F, D] matrix, W1's rows first; the intermediate stays in
  full precision (fp64 here).
* Output: y = g_a y_a + g_b y_b.  Only the two selected experts' weights
  are used.
"""

import numpy as np

from .matvec import gemv_int8, gemv_int8_f64x


def softmax(logits):
    """softmax in fp64 (max-shifted, which leaves the value unchanged)."""
    l = np.asarray(logits, np.float64)
    e = np.exp(l - np.max(l))
    return e / np.sum(e)


def top2(probs):
    """Indices of the two largest entries; equal values -> lower index first."""
    p = np.asarray(probs, np.float64)
    order = sorted(range(len(p)), key=lambda i: (-p[i], i))
    return order[0], order[1]


def route_top2(logits):
    """(selected experts (a, b), renormalised gates (g_a, g_b)) in fp64."""
    p = softmax(logits)
    a, b = top2(p)
    den = p[a] + p[b]
    return (a, b), (p[a] / den, p[b] / den)


def silu(t):
    """silu(t) = t * sigmoid(t) = t / (1 + exp(-t)), fp64."""
    t = np.asarray(t, np.float64)
    return t / (1.0 + np.exp(-t))


def expert_ffn(x_bits, w13_q, w13_s, w2_q, w2_s):
    """One expert's SwiGLU FFN on bf16 activations, fp64 throughout."""
    f = w2_q.shape[1]
    h = gemv_int8(x_bits, w13_q, w13_s)
    a = silu(h[:f]) * h[f:]
    return gemv_int8_f64x(a, w2_q, w2_s)


def moe_top2(x_bits, logits, w13_q, w13_s, w2_q, w2_s):
    """Top-2 MoE decode for one token.

    x_bits [D] bf16 bits; logits [E] fp32; w13_q [E, 2F, D] int8 with
    w13_s [E, 2F] bf16 bits; w2_q [E, D, F] int8 with w2_s [E, D] bf16 bits.
    Returns (y fp64 [D], (a, b), (g_a, g_b)).
    """
    (a, b), (ga, gb) = route_top2(logits)
    ya = expert_ffn(x_bits, w13_q[a], w13_s[a], w2_q[a], w2_s[a])
    yb = expert_ffn(x_bits, w13_q[b], w13_s[b], w2_q[b], w2_s[b])
    return ga * ya + gb * yb, (a, b), (ga, gb)
