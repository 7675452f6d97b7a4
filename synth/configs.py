"""Linear-layer shapes of the decode workloads (no arithmetic).

Each workload is the set of linear layers one batch-1 decode step applies,
W stored [N_out, K_in]:

* Llama-2-7B: 32 layers of {wqkv 4096->12288, wo 4096->4096,
  w1|w3 fused 4096->22016, w2 11008->4096} plus lm_head 4096->32000.
* Llama-3.1-8B: 32 layers of {wqkv 4096->6144, wo 4096->4096,
  w1|w3 4096->28672, w2 14336->4096} plus lm_head 4096->128256.
* Llama-3.1-70B: 80 layers of {wqkv 8192->10240, wo 8192->8192,
  w1|w3 8192->57344, w2 28672->8192} plus lm_head 8192->128256.
* Llama-2-70B: the same layers with lm_head 8192->32000.
* Mixtral-8x7B MoE: 32 layers of 8 experts, each {w1|w3 4096->28672,
  w2 14336->4096}.

The pages benchmark these model families at batch 1 (gittoolsai "gpt-fast"
README mirror, benchmark table "基准测试" and section "Mixtral 8x7B").

Tensor-parallel shards (the same README, tables "张量并行" and "张量并行 +
量化"; awesome-repositories "meta-pytorch/gpt-fast", tag "Linear Layer
Sharding"): with P GPUs each GPU holds 1/P of every layer.  wqkv and w1|w3
are split by output rows (column-parallel; w1 and w3 split alike, so the
fused matrix keeps 2 ffn/P rows), wo and w2 by input columns
(row-parallel: each GPU's K is dim/P or ffn/P); lm_head stays whole on
every GPU, as the pages' per-GPU bandwidth figures imply.
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Model:
    name: str
    dim: int
    qkv: int
    ffn: int
    vocab: int
    layers: int


LLAMA2_7B = Model("llama-2-7b", 4096, 12288, 11008, 32000, 32)
LLAMA31_8B = Model("llama-3.1-8b", 4096, 6144, 14336, 128256, 32)
LLAMA31_70B = Model("llama-3.1-70b", 8192, 10240, 28672, 128256, 80)
LLAMA2_70B = Model("llama-2-70b", 8192, 10240, 28672, 32000, 80)


@dataclass(frozen=True)
class MoEModel:
    name: str
    dim: int
    ffn: int
    experts: int
    top: int
    layers: int


MIXTRAL_8X7B = MoEModel("mixtral-8x7b", 4096, 14336, 8, 2, 32)

# matrix ids inside one layer (used in seeds)
WQKV, WO, W13, W2, LM_HEAD = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Matrix:
    name: str
    layer: int
    mid: int
    n: int
    k: int

    @property
    def weights(self):
        return self.n * self.k


def layer_matrices(model, layer, tp=1):
    """One layer's four linears; with tp > 1, one GPU's shard of each."""
    d = model.dim
    for v in (model.qkv, d, model.ffn):
        if v % tp:
            raise ValueError(f"{model.name}: {v} does not split {tp} ways")
    return [
        Matrix("wqkv", layer, WQKV, model.qkv // tp, d),
        Matrix("wo", layer, WO, d, d // tp),
        Matrix("w13", layer, W13, 2 * model.ffn // tp, d),
        Matrix("w2", layer, W2, d, model.ffn // tp),
    ]


def linear_set(model, layers=None, tp=1):
    """All linears of one decode step: layers x 4 matrices + lm_head (with
    tp > 1: one GPU's shards, lm_head whole)."""
    n_layers = model.layers if layers is None else layers
    out = []
    for layer in range(n_layers):
        out += layer_matrices(model, layer, tp)
    out.append(Matrix("lm_head", model.layers, LM_HEAD, model.vocab, model.dim))
    return out


def distinct_shapes(model, tp=1):
    """One matrix of each distinct shape (layer 0 and lm_head)."""
    return layer_matrices(model, 0, tp) + [Matrix("lm_head", model.layers, LM_HEAD, model.vocab, model.dim)]
