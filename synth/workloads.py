"""The measured workloads: which linears, which format, which inputs (no arithmetic).

Each workload is one batch-1 decode step (or one speculative-verify pass) of
a model family the pages benchmark, with synthetic N(0, sigma) weights and
N(0, 1) bf16 activations standing in for trained checkpoints:

  int8-4096        one int8 per-row GEMV, W [4096, 4096] N(0, 0.02), seed 0;
                   a step sweeps 64 resident copies of it
  llama2-7b-int4   Llama-2-7B linear set, int4 G=32          (129 matvecs)
  llama2-7b-int4g128  the same weights, int4 with groups of 128 inputs
  llama2-7b-int4pc    the same weights, int4 with one group per output row
  llama2-7b-bf16 / llama2-7b-int8 / llama3.1-8b-bf16 / llama3.1-8b-int8
  llama3.1-70b-int4-m5  Llama-3.1-70B set, int4 G=32, 5 tokens per pass,
                        W N(0, 0.015)                       (321 matmuls)
  llama3.1-70b-int8-m5  the same weights in int8, 5 tokens per pass
  llama3.1-70b-int8     the same weights in int8, batch 1 (one token)
  llama3.1-70b-int4-m2 / -m3, llama3.1-70b-int8-m2 / -m3   2 and 3 tokens per pass
  llama2-70b-int8 / llama2-70b-int4   Llama-2-70B set, batch 1
  mixtral-int8     Mixtral-8x7B MoE, 32 layers x 8 int8 experts, top-2
  <set>-tp2 / -tp4 / -tp8   one GPU's shard of the set under P-way tensor
                   parallelism (Llama-2-7B int4 and int8, Llama-3.1-70B int4
                   at 5 tokens): column-parallel wqkv and w1|w3 keep 1/P of
                   their rows, row-parallel wo and w2 1/P of their inputs,
                   lm_head whole

Generators are keyed by (workload id, layer, matrix id, role) so every
matrix has its own reproducible values; the key scheme is in ``synth.gen``.
"""

from dataclasses import dataclass

from .configs import LLAMA2_7B, LLAMA2_70B, LLAMA31_8B, LLAMA31_70B, MIXTRAL_8X7B, Matrix, linear_set
from .gen import ROLE_W, ROLE_X, ROLE_LOGITS, device_normal, device_bf16_normal, host_normal, host_bf16_normal


COPIES = 64


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    fmt: str
    m: int
    sigma: float
    model: object
    note: str = ""
    tp: int = 1

    def matrices(self, layers=None):
        if self.model is None:
            # 64 resident copies of the one seed-0 matrix (same values, distinct
            # addresses): 1.07 GB per sweep, so the 256 MB Infinity Cache cannot
            # serve a repeat and every launch streams from HBM
            n = COPIES if layers is None else 1
            return [Matrix("w", 0, 0, 4096, 4096) for _ in range(n)]
        return linear_set(self.model, layers, self.tp)


WORKLOADS = {w.name: w for w in [
    Workload("int8-4096", 1, "int8", 1, 0.02, None, "single int8 GEMV 4096x4096, seed 0"),
    Workload("llama2-7b-int4", 2, "int4g32", 1, 0.02, LLAMA2_7B),
    Workload("llama2-7b-int4g128", 2, "int4g128", 1, 0.02, LLAMA2_7B),
    Workload("llama2-7b-int4pc", 2, "int4pc", 1, 0.02, LLAMA2_7B),
    Workload("llama2-7b-bf16", 3, "bf16", 1, 0.02, LLAMA2_7B),
    Workload("llama2-7b-int8", 3, "int8", 1, 0.02, LLAMA2_7B),
    Workload("llama3.1-8b-bf16", 6, "bf16", 1, 0.02, LLAMA31_8B),
    Workload("llama3.1-8b-int8", 6, "int8", 1, 0.02, LLAMA31_8B),
    Workload("llama3.1-70b-int4-m5", 4, "int4g32", 5, 0.015, LLAMA31_70B),
    Workload("llama3.1-70b-int8-m5", 4, "int8", 5, 0.015, LLAMA31_70B),
    Workload("llama3.1-70b-int8", 4, "int8", 1, 0.015, LLAMA31_70B),
    # the same sets verifying 2 and 3 draft tokens
    Workload("llama3.1-70b-int4-m2", 4, "int4g32", 2, 0.015, LLAMA31_70B),
    Workload("llama3.1-70b-int4-m3", 4, "int4g32", 3, 0.015, LLAMA31_70B),
    Workload("llama3.1-70b-int8-m2", 4, "int8", 2, 0.015, LLAMA31_70B),
    Workload("llama3.1-70b-int8-m3", 4, "int8", 3, 0.015, LLAMA31_70B),
    Workload("llama2-70b-int8", 7, "int8", 1, 0.015, LLAMA2_70B),
    Workload("llama2-70b-int4", 7, "int4g32", 1, 0.015, LLAMA2_70B),
    Workload("mixtral-int8", 5, "int8", 1, 0.02, MIXTRAL_8X7B),
] + [
    # one GPU's shard under P-way tensor parallelism
    Workload(f"{base}-tp{p}", wid, fmt, m, sigma, model, f"{p}-way tensor-parallel shard", p)
    for base, wid, fmt, m, sigma, model in [("llama2-7b-int4", 2, "int4g32", 1, 0.02, LLAMA2_7B),
                                            ("llama2-7b-int8", 3, "int8", 1, 0.02, LLAMA2_7B),
                                            ("llama3.1-70b-int4-m5", 4, "int4g32", 5, 0.015, LLAMA31_70B)]
    for p in (2, 4, 8)
]}


def gen_w_device(wl, device="cuda"):
    def gen(n, k, mat):
        return device_normal((n, k), wl.sigma, device, wl.wid, mat.layer, mat.mid, ROLE_W)
    return gen


def gen_x_device(wl, device="cuda"):
    def gen(m, k, mat):
        t = device_bf16_normal((m, k), device, wl.wid, mat.layer, mat.mid, ROLE_X)
        return t[0] if m == 1 else t
    return gen


def expert_key(wl, layer, expert, which):
    """Key of a MoE expert matrix: which = 0 for w1|w3, 1 for w2."""
    return (wl.wid, layer, 16 + 2 * expert + which, ROLE_W)


def logits_key(wl, layer):
    return (wl.wid, layer, 0, ROLE_LOGITS)


def moe_x_key(wl, layer):
    return (wl.wid, layer, 0, ROLE_X)


def host_int8_4096():
    """The single-GEMV workload on the host: W [4096, 4096] N(0, 0.02), x bf16, seed 0."""
    w = host_normal((4096, 4096), 0.02, 0)
    x = host_bf16_normal((4096,), 0, 1)
    return w, x
